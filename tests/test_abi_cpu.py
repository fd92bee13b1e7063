"""CPU checks of the C-ABI library: it loads, exports what the header
declares, and rejects bad arguments on the host before touching a GPU.

No call here launches work: each one fails argument validation, which runs
before any HIP call, or is a pure host query (workspace size, plan).
"""
import ctypes
import os
import re

import pytest

from gqa_kv_cache_decode_amd import _lib, build

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gqa_decode.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB_PATH):
        build.build()
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = _declared()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_binding_signatures_match_the_header():
    # the ctypes argument list of every function has the header's parameter count and kinds
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    kinds = {"ptr": ctypes.c_void_p, "int": ctypes.c_int, "float": ctypes.c_float, "size_t": ctypes.c_size_t}
    for name, params in re.findall(r"\b(gqa_\w+)\s*\(([^)]*)\)\s*;", text):
        params = [x.strip() for x in params.split(",") if x.strip() and x.strip() != "void"]
        want = []
        for prm in params:
            if "*" in prm:
                want.append(kinds["ptr"])
            elif prm.startswith("size_t"):
                want.append(kinds["size_t"])
            elif prm.startswith("float"):
                want.append(kinds["float"])
            else:
                want.append(kinds["int"])
        got = [ctypes.c_void_p if (t is ctypes.c_void_p or issubclass(t, ctypes._Pointer)) else t
               for t in _lib.SIGNATURES[name][1]]
        assert got == want, name


def test_header_status_codes_match_binding():
    text = open(HEADER).read()
    codes = dict(re.findall(r"#define (GQA_\w+) \(?(-?\d+)\)?", text))
    assert int(codes["GQA_OK"]) == _lib.OK
    for code, name in _lib.ERROR_NAMES.items():
        assert int(codes[name]) == code
    assert int(codes["GQA_PATH_MATRIX"]) == _lib.PATH_MATRIX
    assert int(codes["GQA_DTYPE_BF16"]) == _lib.BF16


def _attn(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, b=2, h=8, g=2, dk=128, dv=128, cap=100,
             max_len=50, scale=0.1, dtype=_lib.BF16, ws=FAKE, ws_bytes=1 << 30, stream=None, path=0, wgs=0)
    a.update(kw)
    return lib.gqa_decode_attention_ex(a["out"], a["q"], a["k"], a["v"], a["lens"], a["b"], a["h"], a["g"],
                                       a["dk"], a["dv"], a["cap"], a["max_len"], a["scale"], a["dtype"],
                                       a["ws"], a["ws_bytes"], a["stream"], a["path"], a["wgs"])


@pytest.mark.parametrize("kw,code", [
    (dict(h=8, g=3), _lib.ERR_GROUPS),
    (dict(h=28, g=8), _lib.ERR_GROUPS),
    (dict(out=None), _lib.ERR_ARG),
    (dict(lens=None), _lib.ERR_ARG),
    (dict(b=0), _lib.ERR_ARG),
    (dict(b=70000), _lib.ERR_ARG),
    (dict(g=0), _lib.ERR_ARG),
    (dict(max_len=-1), _lib.ERR_ARG),
    (dict(dk=96, dv=96), _lib.ERR_UNSUPPORTED),
    (dict(dk=128, dv=64), _lib.ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.ERR_UNSUPPORTED),
    (dict(max_len=101), _lib.ERR_CAPACITY),
    (dict(ws=None), _lib.ERR_WORKSPACE),
    (dict(ws_bytes=16), _lib.ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x1010)), _lib.ERR_ARG),
    (dict(wgs=-1), _lib.ERR_UNSUPPORTED),
    (dict(wgs=2049), _lib.ERR_UNSUPPORTED),
    (dict(path=9), _lib.ERR_UNSUPPORTED),
    (dict(path=_lib.PATH_MATRIX, dtype=_lib.F32), _lib.ERR_UNSUPPORTED),
    (dict(path=_lib.PATH_MATRIX, dk=64, dv=64), _lib.ERR_UNSUPPORTED),
    (dict(path=_lib.PATH_MATRIX, h=130, g=2), _lib.ERR_UNSUPPORTED),
])
def test_decode_rejects(lib, kw, code):
    assert _attn(lib, **kw) == code
    assert lib.gqa_last_error().decode() != ""


def test_append_rejects(lib):
    def call(**kw):
        a = dict(k=FAKE, v=FAKE, kn=FAKE, vn=FAKE, lens=FAKE, b=4, g=2, dk=16, dv=16, cap=10,
                 max_len=9, dtype=_lib.F32)
        a.update(kw)
        return lib.gqa_kv_append(a["k"], a["v"], a["kn"], a["vn"], a["lens"], a["b"], a["g"], a["dk"],
                                 a["dv"], a["cap"], a["max_len"], a["dtype"], None)
    assert call(max_len=10) == _lib.ERR_CAPACITY
    assert "cap" in lib.gqa_last_error().decode()
    assert call(kn=None) == _lib.ERR_ARG
    assert call(cap=0) == _lib.ERR_ARG
    assert call(b=-1) == _lib.ERR_ARG
    assert call(dtype=3) == _lib.ERR_UNSUPPORTED


def test_workspace_size(lib):
    ws = lib.gqa_decode_workspace_size
    n = ws(16, 64, 8, 128, 128, 8256, _lib.BF16)
    # tickets + two partial slots (m, l, o for a group of 8 heads) per persistent workgroup
    assert n >= 16 * 64 * 4 + 2048 * 2 * 8 * (128 + 2) * 4
    assert n % 256 == 0
    assert ws(16, 64, 8, 128, 128, 100, _lib.BF16) == n  # independent of the length
    # groups smaller than the vector head block are sized for the block (G = 3 -> 4 heads)
    assert ws(1, 12, 4, 128, 128, 10, _lib.BF16) >= 2048 * 2 * 4 * 130 * 4
    assert ws(16, 64, 7, 128, 128, 100, _lib.BF16) == 0  # h % g != 0
    assert ws(16, 64, 8, 128, 128, -1, _lib.BF16) == 0
    assert ws(1, 1, 1, 16, 16, 0, _lib.F32) > 0


def test_workspace_size_monotone(lib):
    # a buffer sized for one shape must serve every smaller shape: the size
    # never decreases as b, h (at fixed h/g) or d_v grow, also across the
    # b*h = 8192 boundary where the tickets stop being padded to 128 bytes
    ws = lib.gqa_decode_workspace_size
    shapes = [(b, G * g, g, d) for b in (1, 7, 64, 128, 129, 256, 1024) for g in (1, 2, 8)
              for G in (1, 4, 8, 64) for d in (16, 128) if G * g <= 4096]
    for (b, h, g, d) in shapes:
        n = ws(b, h, g, d, d, 100, _lib.BF16)
        assert n > 0 and n % 256 == 0
        bh = b * h
        tickets = 32 * bh if bh <= 8192 else max(bh, 262144)
        assert n >= 4 * tickets + 256
        for (b2, h2, g2, d2) in shapes:
            if b2 <= b and h2 <= h and h2 // g2 <= h // g and d2 <= d:
                assert ws(b2, h2, g2, d2, d2, 100, _lib.BF16) <= n, ((b, h, g, d), (b2, h2, g2, d2))


def test_plan_choices(lib):
    def plan(b, h, g, d, cap, max_len, dtype, path=0, wgs=0):
        p, c = ctypes.c_int(), ctypes.c_int()
        rc = lib.gqa_decode_plan(b, h, g, d, d, cap, max_len, dtype, path, wgs, ctypes.byref(p), ctypes.byref(c))
        assert rc == _lib.OK, lib.gqa_last_error()
        return p.value, c.value
    M = _lib.MERGE_INLINE | _lib.MERGE_KERNEL
    # the Llama-3-70B shape: the matrix path's one-block streaming kernel, merges inside the launch
    assert plan(16, 64, 8, 128, 8256, 8193, _lib.BF16)[0] == _lib.PATH_MATRIX | _lib.MERGE_INLINE | _lib.PLAN_STREAM
    assert plan(64, 28, 4, 128, 2112, 2080, _lib.BF16)[0] & _lib.PLAN_STREAM  # the Qwen2.5-7B shape too
    # up to 64 heads per KV head (two or four column blocks) as well
    assert plan(16, 64, 2, 128, 2112, 2080, _lib.BF16)[0] & _lib.PLAN_STREAM
    assert plan(16, 24, 1, 128, 2112, 2080, _lib.BF16)[0] & _lib.PLAN_STREAM
    assert plan(16, 64, 1, 128, 2112, 2080, _lib.BF16)[0] & _lib.PLAN_STREAM
    # 64 heads per KV head: merged inline up to three parts per segment (two waves of 32 heads), else
    # by a second launch
    assert plan(64, 128, 2, 128, 2112, 2048, _lib.BF16)[0] == _lib.PATH_MATRIX | _lib.MERGE_INLINE | _lib.PLAN_STREAM
    assert plan(64, 64, 1, 128, 2112, 2048, _lib.BF16)[0] == _lib.PATH_MATRIX | _lib.MERGE_KERNEL | _lib.PLAN_STREAM
    # past 64 sequences: the unit kernels
    assert not plan(65, 64, 8, 128, 2112, 2080, _lib.BF16)[0] & _lib.PLAN_STREAM
    assert not plan(65, 64, 1, 128, 2112, 2080, _lib.BF16)[0] & _lib.PLAN_STREAM
    M = M | _lib.PLAN_STREAM
    # few long segments with 32 heads per KV head: merged by a second launch
    S = _lib.PATH_MATRIX | _lib.MERGE_KERNEL | _lib.PLAN_STREAM
    assert plan(8, 32, 1, 128, 4160, 4097, _lib.BF16)[0] == S
    assert plan(4, 32, 1, 128, 32832, 32769, _lib.BF16)[0] == S
    assert plan(4, 32, 32, 128, 32832, 32769, _lib.BF16)[0] & ~M == _lib.PATH_VECTOR  # one head per KV head
    assert plan(2, 4, 2, 16, 128, 65, _lib.F32)[0] & ~M == _lib.PATH_VECTOR
    for args in [(16, 64, 8, 128, 8256, 8193, _lib.BF16), (2, 4, 2, 16, 128, 65, _lib.F32),
                 (64, 28, 4, 128, 2112, 2080, _lib.BF16)]:
        _, c = plan(*args)
        assert 1 <= c <= 2048
    assert plan(16, 64, 8, 128, 8256, 8193, _lib.BF16, path=_lib.PATH_VECTOR, wgs=77)[1] == 77
    # forced merge modes are kept; both flags at once are rejected
    for flag in (_lib.MERGE_INLINE, _lib.MERGE_KERNEL):
        assert plan(8, 32, 1, 128, 4160, 4097, _lib.BF16, path=_lib.PATH_MATRIX | flag)[0] & ~_lib.PLAN_STREAM == \
            _lib.PATH_MATRIX | flag
        assert plan(2, 4, 2, 16, 128, 65, _lib.F32, path=flag)[0] == _lib.PATH_VECTOR | flag
    p, c = ctypes.c_int(), ctypes.c_int()
    assert lib.gqa_decode_plan(8, 32, 1, 128, 128, 4160, 4097, _lib.BF16, M, 0, ctypes.byref(p),
                               ctypes.byref(c)) == _lib.ERR_UNSUPPORTED


def test_plan_spread_merge(lib):
    def plan(b, h, g, d, cap, max_len, dtype, path, wgs=0):
        p, c = ctypes.c_int(), ctypes.c_int()
        rc = lib.gqa_decode_plan(b, h, g, d, d, cap, max_len, dtype, path, wgs, ctypes.byref(p), ctypes.byref(c))
        return rc, p.value
    # kept where the stream kernel runs, whatever the grid
    for args in [(8, 32, 1, 128, 4160, 4097), (16, 64, 8, 128, 8256, 8193), (2, 192, 3, 128, 300, 200)]:
        for wgs in (0, 1, 2048):
            rc, p = plan(*args, _lib.BF16, _lib.PATH_MATRIX | _lib.MERGE_SPREAD, wgs)
            assert rc == _lib.OK and p == _lib.PATH_MATRIX | _lib.MERGE_SPREAD | _lib.PLAN_STREAM, (args, wgs)
    # refused elsewhere: more than 64 sequences, fp32, other head dims, two heads per KV head
    for args, dt in [((65, 32, 1, 128, 300, 200), _lib.BF16), ((2, 4, 2, 16, 128, 65), _lib.F32),
                     ((8, 32, 1, 64, 300, 200), _lib.BF16), ((8, 2, 1, 128, 300, 200), _lib.BF16)]:
        assert plan(*args, dt, _lib.MERGE_SPREAD)[0] == _lib.ERR_UNSUPPORTED, args
    # with another merge flag
    for other in (_lib.MERGE_INLINE, _lib.MERGE_KERNEL):
        assert plan(8, 32, 1, 128, 4160, 4097, _lib.BF16, _lib.MERGE_SPREAD | other)[0] == _lib.ERR_UNSUPPORTED


def test_step_rejects(lib):
    def call(**kw):
        a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, k=FAKE, v=FAKE, lens=FAKE, b=2, h=8, g=2, dk=128, dv=128,
                 cap=100, max_len=50, dtype=_lib.BF16, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.gqa_decode_step(a["out"], a["q"], a["kn"], a["vn"], a["k"], a["v"], a["lens"], a["b"], a["h"],
                                   a["g"], a["dk"], a["dv"], a["cap"], a["max_len"], 0.1, a["dtype"], a["ws"],
                                   a["ws_bytes"], None)
    assert call(max_len=100) == _lib.ERR_CAPACITY  # no room for the appended token
    assert call(kn=None) == _lib.ERR_ARG
    assert call(lens=None) == _lib.ERR_ARG
    assert call(h=8, g=3) == _lib.ERR_GROUPS
    assert call(dk=96, dv=96) == _lib.ERR_UNSUPPORTED
    assert call(ws_bytes=8) == _lib.ERR_WORKSPACE
    assert call(max_len=-2) == _lib.ERR_ARG


def test_linear_rejects(lib):
    def call(**kw):
        a = dict(y=FAKE, x=FAKE, w=FAKE, rows=16, n_in=64, n_out=32, dtype=_lib.BF16)
        a.update(kw)
        return lib.gqa_linear(a["y"], a["x"], a["w"], a["rows"], a["n_in"], a["n_out"], a["dtype"], None)
    assert call(dtype=_lib.F32) == _lib.ERR_UNSUPPORTED
    assert call(rows=65) == _lib.ERR_UNSUPPORTED
    assert call(rows=0) == _lib.ERR_UNSUPPORTED
    assert call(n_in=12) == _lib.ERR_UNSUPPORTED
    assert call(n_out=0) == _lib.ERR_ARG
    assert call(w=None) == _lib.ERR_ARG
    assert call(x=ctypes.c_void_p(0x1008)) == _lib.ERR_ARG  # not 16-byte aligned
    assert lib.gqa_last_error().decode() != ""


def test_decode_layer_rejects(lib):
    def call(**kw):
        a = dict(b=16, h=64, g=8, d_model=8192, d=128, cap=100, max_len=50, dtype=_lib.BF16, ws=FAKE,
                 ws_bytes=1 << 30, x=FAKE)
        a.update(kw)
        return lib.gqa_decode_layer(FAKE, a["x"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    a["b"], a["h"], a["g"], a["d_model"], a["d"], a["d"], a["cap"], a["max_len"],
                                    ctypes.c_float(0.1), a["dtype"], a["ws"], a["ws_bytes"], None)
    assert call(dtype=_lib.F32) == _lib.ERR_UNSUPPORTED
    assert call(b=65) == _lib.ERR_UNSUPPORTED
    assert call(d_model=100) == _lib.ERR_UNSUPPORTED
    assert call(d_model=0) == _lib.ERR_ARG
    assert call(x=None) == _lib.ERR_ARG
    assert call(max_len=100) == _lib.ERR_CAPACITY
    assert call(h=60) == _lib.ERR_GROUPS
    assert call(ws_bytes=64) == _lib.ERR_WORKSPACE
    assert call(d=96) == _lib.ERR_UNSUPPORTED


def test_fold_rejects(lib):
    FAKE2 = ctypes.c_void_p(1 << 40)  # far from FAKE: no overlap

    def call(**kw):
        a = dict(dst=FAKE2, src=FAKE, lens=None, b=2, g_src=8, g_dst=2, cap_src=64, cap_dst=64, d=128, rows=64,
                 dtype=_lib.BF16)
        a.update(kw)
        return lib.gqa_fold_kv_heads(a["dst"], a["src"], a["lens"], a["b"], a["g_src"], a["g_dst"], a["cap_src"],
                                     a["cap_dst"], a["d"], a["rows"], a["dtype"], None)
    assert call(rows=0) == _lib.OK  # nothing to fold: nothing is enqueued
    assert call(g_dst=3, rows=0) == _lib.ERR_GROUPS
    assert call(d=12, rows=0) == _lib.ERR_UNSUPPORTED
    assert call(dtype=7, rows=0) == _lib.ERR_UNSUPPORTED
    assert call(rows=65) == _lib.ERR_CAPACITY
    assert call(cap_dst=32) == _lib.ERR_CAPACITY
    assert call(rows=-1) == _lib.ERR_ARG
    assert call(src=None) == _lib.ERR_ARG
    assert call(b=0) == _lib.ERR_ARG
    assert call(dst=FAKE, rows=0) == _lib.ERR_ARG  # the same buffer: overlap
    assert call(dst=ctypes.c_void_p((1 << 40) + 8), rows=0) == _lib.ERR_ARG  # not 16-byte aligned
    assert lib.gqa_last_error().decode() != ""


def test_read_bandwidth_rejects(lib):
    def call(src=FAKE, nbytes=1 << 20, sink=FAKE, wgs=256):
        return lib.gqa_read_bandwidth(src, nbytes, sink, wgs, None)
    assert call(src=None) == _lib.ERR_ARG
    assert call(sink=None) == _lib.ERR_ARG
    for wgs in (0, -1, 2049):
        assert call(wgs=wgs) == _lib.ERR_ARG, wgs
    assert call(nbytes=(1 << 20) + 8) == _lib.ERR_ARG                # not a multiple of 16
    assert call(src=ctypes.c_void_p(0x1008)) == _lib.ERR_ARG         # not 16-byte aligned
    assert call(nbytes=(1 << 31) + 16, wgs=1) == _lib.ERR_ARG         # more than 2 GiB for one workgroup
    assert b"gqa_read_bandwidth" in lib.gqa_last_error()


def test_paged_rejects(lib):
    FAKE2 = ctypes.c_void_p(1 << 40)

    def step(**kw):
        a = dict(table=FAKE2, b=4, h=8, g=2, d=128, bs=64, mb=4, nb=16, max_len=100, dtype=_lib.BF16, ws_bytes=1 << 30)
        a.update(kw)
        return lib.gqa_decode_step_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], a["b"], a["h"], a["g"],
                                         a["d"], a["d"], a["bs"], a["mb"], a["nb"], a["max_len"], ctypes.c_float(0.1),
                                         a["dtype"], FAKE, a["ws_bytes"], None)

    def attend(**kw):
        a = dict(table=FAKE2, b=4, h=8, g=2, d=128, bs=64, mb=4, nb=16, max_len=100, ws_bytes=1 << 30)
        a.update(kw)
        return lib.gqa_decode_attention_paged(FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], a["b"], a["h"], a["g"],
                                              a["d"], a["d"], a["bs"], a["mb"], a["nb"], a["max_len"],
                                              ctypes.c_float(0.1), _lib.BF16, FAKE, a["ws_bytes"], None)

    def append(**kw):
        a = dict(table=FAKE2, b=4, bs=64, mb=4, nb=16, max_len=100)
        a.update(kw)
        return lib.gqa_kv_append_paged(FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], a["b"], 2, 128, 128, a["bs"],
                                       a["mb"], a["nb"], a["max_len"], _lib.BF16, None)

    for call in (step, attend, append):
        assert call(table=None) == _lib.ERR_ARG
        assert call(bs=16) == _lib.ERR_UNSUPPORTED    # below one 32-position tile
        assert call(bs=96) == _lib.ERR_UNSUPPORTED    # not a power of two
        assert call(mb=0) == _lib.ERR_ARG
        assert call(nb=0) == _lib.ERR_ARG
    assert step(max_len=256) == _lib.ERR_CAPACITY       # 4 blocks of 64: the append needs position 256
    assert append(max_len=256) == _lib.ERR_CAPACITY
    assert attend(max_len=257) == _lib.ERR_CAPACITY
    assert step(h=6, g=4) == _lib.ERR_GROUPS
    assert step(d=48) == _lib.ERR_UNSUPPORTED
    assert step(ws_bytes=64) == _lib.ERR_WORKSPACE
    assert lib.gqa_last_error().decode() != ""


def test_multi_rejects_on_the_host(lib):
    def attend(**kw):
        a = dict(b=4, n=2, h=64, g=8, d=128, cap=100, max_len=60, dtype=_lib.BF16, ws_bytes=1 << 30)
        a.update(kw)
        return lib.gqa_decode_attention_multi(FAKE, FAKE, FAKE, FAKE, FAKE, a["b"], a["n"], a["h"], a["g"], a["d"],
                                              a["d"], a["cap"], a["max_len"], ctypes.c_float(0.1), a["dtype"], FAKE,
                                              a["ws_bytes"], None)

    def step(**kw):
        a = dict(b=4, n=2, h=64, g=8, d=128, cap=100, max_len=60, dtype=_lib.BF16, ws_bytes=1 << 30)
        a.update(kw)
        return lib.gqa_decode_step_multi(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["b"], a["n"], a["h"], a["g"],
                                         a["d"], a["d"], a["cap"], a["max_len"], ctypes.c_float(0.1), a["dtype"], FAKE,
                                         a["ws_bytes"], None)
    for call in (attend, step):
        assert call(n=0) == _lib.ERR_ARG
        assert call(n=65) == _lib.ERR_ARG
        assert call(n=64, h=128, g=8) == _lib.ERR_ARG  # 64 x 128 query rows > 4096
        assert call(dtype=7) == _lib.ERR_UNSUPPORTED
        assert call(d=48) == _lib.ERR_UNSUPPORTED
        assert call(h=60) == _lib.ERR_GROUPS
        assert call(ws_bytes=64) == _lib.ERR_WORKSPACE
    assert attend(max_len=101) == _lib.ERR_CAPACITY
    assert step(max_len=99) == _lib.ERR_CAPACITY       # 99 + 2 > 100
    assert lib.gqa_kv_append_multi(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 3, 8, 128, 128, 100, 98, _lib.BF16,
                                   None) == _lib.ERR_CAPACITY
    # the multi-token workspace is that of a one-token call with n * h heads
    assert lib.gqa_decode_multi_workspace_size(4, 2, 64, 8, 128, 128, _lib.BF16) == \
        lib.gqa_decode_workspace_size(4, 128, 8, 128, 128, 0, _lib.BF16)
    assert lib.gqa_decode_multi_workspace_size(4, 0, 64, 8, 128, 128, _lib.BF16) == 0


def test_multi_paged_rejects_on_the_host(lib):
    FAKE2 = ctypes.c_void_p(1 << 40)
    base = dict(table=FAKE2, b=4, n=2, h=64, g=8, d=128, bs=64, mb=4, nb=16, max_len=100, dtype=_lib.BF16,
                ws_bytes=1 << 30)

    def attend(**kw):
        a = dict(base, **kw)
        return lib.gqa_decode_attention_multi_paged(FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], a["b"], a["n"], a["h"],
                                                    a["g"], a["d"], a["d"], a["bs"], a["mb"], a["nb"], a["max_len"],
                                                    ctypes.c_float(0.1), a["dtype"], FAKE, a["ws_bytes"], None)

    def step(**kw):
        a = dict(base, **kw)
        return lib.gqa_decode_step_multi_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], a["b"], a["n"],
                                               a["h"], a["g"], a["d"], a["d"], a["bs"], a["mb"], a["nb"], a["max_len"],
                                               ctypes.c_float(0.1), a["dtype"], FAKE, a["ws_bytes"], None)

    def append(**kw):
        a = dict(base, **kw)
        return lib.gqa_kv_append_multi_paged(FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], a["b"], a["n"], a["g"], a["d"],
                                             a["d"], a["bs"], a["mb"], a["nb"], a["max_len"], a["dtype"], None)

    for call in (attend, step, append):
        assert call(table=None) == _lib.ERR_ARG
        assert call(bs=16) == _lib.ERR_UNSUPPORTED      # below one 32-position tile
        assert call(bs=96) == _lib.ERR_UNSUPPORTED      # not a power of two
        assert call(mb=0) == _lib.ERR_ARG
        assert call(n=0) == _lib.ERR_ARG
        assert call(n=65) == _lib.ERR_ARG
        assert call(dtype=7) == _lib.ERR_UNSUPPORTED
    for call in (attend, step):
        assert call(n=64, h=128) == _lib.ERR_ARG         # 64 x 128 query rows > 4096
        assert call(h=60) == _lib.ERR_GROUPS
        assert call(d=48) == _lib.ERR_UNSUPPORTED
        assert call(ws_bytes=64) == _lib.ERR_WORKSPACE
    assert attend(max_len=257) == _lib.ERR_CAPACITY      # 4 blocks of 64 positions
    assert step(max_len=255) == _lib.ERR_CAPACITY        # 255 + 2 > 256
    assert append(max_len=255) == _lib.ERR_CAPACITY


def test_static_scratch_step_rejects_on_the_host(lib):
    # the allocation-free step checks everything a workspace call checks, and
    # refuses shapes whose workspace would not fit its 8 MiB array, before any
    # device work (no GPU is needed to reach these codes)
    def step(**kw):
        a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, b=16, h=64, g=8, d=128, cap=8300,
                 max_len=8192, scale=0.088, dtype=_lib.BF16)
        a.update(kw)
        return lib.gqa_decode_step_static(a["out"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["lens"], a["b"],
                                          a["h"], a["g"], a["d"], a["d"], a["cap"], a["max_len"], a["scale"],
                                          a["dtype"], None)
    assert step(q=None) == _lib.ERR_ARG
    assert step(h=60, g=8) == _lib.ERR_GROUPS
    assert step(max_len=8300) == _lib.ERR_CAPACITY
    assert step(d=96) == _lib.ERR_UNSUPPORTED
    # 64 sequences x 4096 heads, 64 heads per KV head: slots, segment table
    # and tickets far beyond 8 MiB
    assert step(b=64, h=4096, g=64, cap=4, max_len=1) == _lib.ERR_WORKSPACE
    assert "static scratch" in lib.gqa_last_error().decode()
