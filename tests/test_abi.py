"""The C ABI on the CPU: the library loads, exports every function include/dg.h
declares, and rejects bad arguments with the documented status codes before it
makes any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


@pytest.fixture(scope="module")
def dg():
    import fp8_block_scaled_scales_amd as dg

    return dg


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_api():
    names = _declared_functions()
    for f in ("dg_gemm_fp8_nt", "dg_query_tile", "dg_strerror", "dg_version", "dg_gemm_fp8_ws", "dg_query_tile_ws"):
        assert f in names


def test_tile_info_layout_matches_header(dg):
    # the ctypes mirror of dg_tile_info: same fields, same order, same size as the C struct
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct dg_tile_info \{(.*?)\} dg_tile_info;", text, flags=re.S).group(1)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        ctype, names = decl.split(None, 1)
        fields += [(n.strip(), ctype) for n in names.split(",")]
    assert [f for f, _ in fields] == [f for f, _ in dg.dg_tile_info._fields_]
    size = {"int": 4, "int64_t": 8}
    assert all(ctypes.sizeof(t) == size[c] for (_, c), (_, t) in zip(fields, dg.dg_tile_info._fields_))
    assert ctypes.sizeof(dg.dg_tile_info) == 48


def test_library_exports_every_declared_symbol(dg):
    lib = ctypes.CDLL(dg.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_race_check_build_exports_every_declared_symbol(dg):
    # the build with extra waits and barriers per pipeline step answers the
    # same host-side calls the same way
    lib = dg.load_library(dg.SYNC_LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.dg_version() == dg.dg_version()
    for M, N, K, g, layout in [(64, 4096, 7168, 128, 0), (64, 512, 7168, 128, 1), (8192, 8192, 8192, 128, 3)]:
        a, b = dg.dg_tile_info(), dg.dg_tile_info()
        assert lib.dg_query_tile_ws(M, N, K, g, layout, ctypes.byref(a)) == 0
        assert dg.lib.dg_query_tile_ws(M, N, K, g, layout, ctypes.byref(b)) == 0
        assert [getattr(a, f) for f, _ in a._fields_] == [getattr(b, f) for f, _ in b._fields_]


def test_status_codes_match_header(dg):
    text = open(HEADER).read()
    for name in ("DG_OK", "DG_EINVAL", "DG_EALIGN", "DG_EUNSUPPORTED", "DG_ELAUNCH", "DG_ESCRATCH"):
        m = re.search(r"#define %s \(?(-?\d+)\)?" % name, text)
        assert m and int(m.group(1)) == getattr(dg, name), name
    assert dg.dg_version() == int(re.search(r"#define DG_VERSION (\d+)", text).group(1))
    m = re.search(r"#define DG_MAX_DIM \(\(1LL << (\d+)\) - (\d+)\)", text)
    assert m and (1 << int(m.group(1))) - int(m.group(2)) == dg.DG_MAX_DIM
    # a 256-row tile of K bytes per row stays inside a 32-bit byte range, and the
    # largest K is a multiple of every g
    assert 256 * dg.DG_MAX_DIM < 1 << 32 and dg.DG_MAX_DIM % 256 == 0


@pytest.mark.parametrize("g", [64, 128, 256])
def test_max_dims_accepted(dg, g):
    mx = dg.DG_MAX_DIM
    for M, N, K in [(256, 256, mx), (2048, 3072, mx), (64, 4096, mx), (mx, 256, 256), (256, mx, 256)]:
        for layout in range(4):
            assert dg.dg_query_tile(M, N, K, g, layout)["grid"] > 0
    with pytest.raises(ValueError):
        dg.dg_query_tile(256, 256, mx + 256, g)


# Fake but aligned, non-null device addresses: the checks below must fail
# before anything dereferences them or calls into HIP.
A, B, SA, SB, OUT = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def _call(dg, a=A, b=B, sa=SA, sb=SB, out=OUT, M=256, N=256, K=256, g=128):
    return dg.lib.dg_gemm_fp8_nt(a, b, sa, sb, out, M, N, K, g, None)


@pytest.mark.parametrize("kw", [dict(a=0), dict(b=0), dict(sa=0), dict(sb=0), dict(out=0),
                                dict(M=0), dict(N=0), dict(K=0), dict(M=-5), dict(K=-128),
                                dict(K=192), dict(K=100, g=64), dict(g=96), dict(g=512), dict(K=384, g=256), dict(g=0),
                                dict(M=(1 << 24) + 1), dict(K=1 << 25), dict(K=1 << 24),
                                dict(N=(1 << 24) - 255)])
def test_einval(dg, kw):
    assert _call(dg, **kw) == dg.DG_EINVAL


@pytest.mark.parametrize("kw", [dict(a=A + 8), dict(b=B + 4), dict(sa=SA + 2), dict(sb=SB + 1), dict(out=OUT + 1)])
def test_ealign(dg, kw):
    assert _call(dg, **kw) == dg.DG_EALIGN


@pytest.mark.parametrize("fa,fb,kw", [(2, 0, {}), (0, -1, {}), (1, 7, {}), (1, 1, dict(K=384, g=256)),
                                      (0, 1, dict(a=0)), (1, 0, dict(g=32))])
def test_fmt_einval(dg, fa, fb, kw):
    args = dict(a=A, b=B, sa=SA, sb=SB, out=OUT, M=256, N=256, K=256, g=128)
    args.update(kw)
    assert dg.lib.dg_gemm_fp8_nt_fmt(args["a"], args["b"], args["sa"], args["sb"], args["out"], args["M"], args["N"],
                                     args["K"], args["g"], fa, fb, None) == dg.DG_EINVAL


@pytest.mark.parametrize("fmt,g,cols", [(2, 128, 256), (-1, 128, 256), (1, 96, 192), (0, 256, 384)])
def test_quantize_einval(dg, fmt, g, cols):
    assert dg.lib.dg_quantize_fp8_blocks(A, 64, cols, g, fmt, B, SA, None) == dg.DG_EINVAL


@pytest.mark.parametrize("act,bias,want", [(3, 0, "DG_EINVAL"), (-1, 0, "DG_EINVAL"), (1, SB + 2, "DG_EALIGN")])
def test_epi_rejects(dg, act, bias, want):
    assert dg.lib.dg_gemm_fp8_nt_epi(A, B, SA, SB, OUT, 256, 256, 256, 128, 0, 0, bias or None, act, None) == \
        getattr(dg, want)


@pytest.mark.parametrize("g,sa_rows,kw,want", [(128, 2, {}, "DG_EINVAL"), (128, 64, {}, "DG_EINVAL"),
                                                (128, 0, {}, "DG_EINVAL"), (64, 128, {}, "DG_EINVAL"),
                                                (256, 1, dict(K=384), "DG_EINVAL"), (128, 1, dict(sa=SA + 2), "DG_EALIGN"),
                                                (128, 1, dict(a=0), "DG_EINVAL"), (128, 1, dict(fa=2), "DG_EINVAL"),
                                                (128, 1, dict(act=5), "DG_EINVAL")])
def test_ex_rejects(dg, g, sa_rows, kw, want):
    args = dict(a=A, sa=SA, K=256, fa=0, act=0)
    args.update(kw)
    assert dg.lib.dg_gemm_fp8_nt_ex(args["a"], B, args["sa"], SB, OUT, 256, 256, args["K"], g, sa_rows, args["fa"], 0,
                                    None, args["act"], None) == getattr(dg, want)


@pytest.mark.parametrize("fmt,g,cols", [(2, 128, 256), (1, 96, 192), (0, 256, 384), (0, 128, 0)])
def test_quantize_rows_einval(dg, fmt, g, cols):
    assert dg.lib.dg_quantize_fp8_rows(A, 64, cols, g, fmt, B, SA, None) == dg.DG_EINVAL


def test_python_binding_checks_row_scale_shapes(dg):
    import torch

    # the tensor checks run before the device check, so CPU tensors reach them
    a = torch.zeros((300, 256), dtype=torch.float8_e4m3fn)
    b = torch.zeros((64, 256), dtype=torch.float8_e4m3fn)
    sb = torch.zeros((1, 2))
    with pytest.raises(ValueError, match="sa has shape"):
        dg.dg_gemm_fp8_nt_ex(a, b, torch.zeros((3, 2)), sb, sa_rows=1)
    with pytest.raises(ValueError, match="sa has shape"):
        dg.dg_gemm_fp8_nt_ex(a, b, torch.zeros((300, 2)), sb)  # per-row factors for a block-scaled call
    with pytest.raises(ValueError, match="sa_rows"):
        dg.dg_gemm_fp8_nt_ex(a, b, torch.zeros((300, 2)), sb, sa_rows=7)
    with pytest.raises(ValueError, match="GPU tensor"):
        dg.dg_gemm_fp8_nt_ex(a, b, torch.zeros((300, 2)), sb, sa_rows=1)  # well-formed, but on the CPU


@pytest.mark.parametrize("layout,M,N,want", [(4, 256, 256, "DG_EINVAL"), (-1, 256, 256, "DG_EINVAL"),
                                              (7, 1000, 256, "DG_EINVAL")])
def test_layout_rejects(dg, layout, M, N, want):
    assert dg.lib.dg_gemm_fp8_layout(A, B, SA, SB, OUT, M, N, 256, 128, layout, 0, 0, None, 0, None) == getattr(dg, want)
    info = dg.dg_tile_info()
    assert dg.lib.dg_query_tile_layout(M, N, 256, 128, layout, ctypes.byref(info)) == getattr(dg, want)


@pytest.mark.parametrize("layout,M,N", [(2, 1000, 256), (3, 1001, 257), (1, 256, 1000), (3, 7, 4095), (1, 64, 4099)])
def test_layout_accepts_any_row_length(dg, layout, M, N):
    # a transposed operand's stored rows (M or N bytes) need not be a multiple of 16 long
    t = dg.dg_query_tile(M, N, 256, 128, layout)
    assert t["grid"] > 0 and t["ksplit"] == 1


@pytest.mark.parametrize("M,N,K,g,layout,tile", [(64, 4096, 7168, 128, 1, (32, 32)), (4096, 7168, 2048, 128, 3, (256, 256)),
                                                 (1008, 3008, 512, 64, 2, (128, 128)), (128, 512, 1024, 256, 3, (32, 32)),
                                                 (2000, 4000, 1024, 128, 1, (256, 128)), (3584, 3584, 512, 256, 2, (256, 256))])
def test_layout_tile_choice(dg, M, N, K, g, layout, tile):
    # transposed layouts: the NT choice, streaming 32x32 tiles for M <= 128, else the 256-row tiles 256 or 128
    # wide or 128x128; without a workspace nothing splits K
    t = dg.dg_query_tile(M, N, K, g, layout)
    assert (t["bm"], t["bn"]) == tile
    assert t["ksplit"] == 1 and t["workspace_bytes"] == 0
    assert dg.dg_query_tile(M, N, K, g, 0) == dg.dg_query_tile(M, N, K, g)


def test_layout_codes_match_header(dg):
    text = open(HEADER).read()
    for name in ("DG_LAYOUT_NT", "DG_LAYOUT_NN", "DG_LAYOUT_TT", "DG_LAYOUT_TN"):
        m = re.search(r"#define %s (\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(dg, name), name


def test_python_binding_checks_layout_shapes(dg):
    import torch

    a_km = torch.zeros((256, 64), dtype=torch.float8_e4m3fn)   # A stored [K, M]
    b_nk = torch.zeros((32, 256), dtype=torch.float8_e4m3fn)   # B stored [N, K]
    sa, sb = torch.zeros((1, 2)), torch.zeros((1, 2))
    with pytest.raises(ValueError, match="b has shape"):
        dg.dg_gemm_fp8_layout(a_km, b_nk, sa, sb, layout=dg.DG_LAYOUT_TN)  # TN wants B [K, N]
    with pytest.raises(ValueError, match="GPU tensor"):
        dg.dg_gemm_fp8_layout(a_km, b_nk, sa, sb, layout=dg.DG_LAYOUT_TT)  # well-formed, but on the CPU
    with pytest.raises(ValueError, match="layout"):
        dg.dg_gemm_fp8_layout(a_km, b_nk, sa, sb, layout=5)


def test_format_codes_match_header(dg):
    text = open(HEADER).read()
    for name in ("DG_FMT_E4M3", "DG_FMT_E5M2", "DG_ACT_NONE", "DG_ACT_RELU", "DG_ACT_GELU", "DG_IN_F32", "DG_IN_BF16",
                 "DG_IN_F16"):
        m = re.search(r"#define %s (\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(dg, name), name


def test_strerror(dg):
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(dg.dg_strerror(code), str) and dg.dg_strerror(code)


@pytest.mark.parametrize("M,N,K,g", [(256, 256, 256, 128), (64, 4096, 7168, 128), (4096, 7168, 2048, 128),
                                     (8192, 8192, 8192, 128), (2000, 4000, 16384, 64), (1, 1, 64, 64)])
def test_query_tile(dg, M, N, K, g):
    t = dg.dg_query_tile(M, N, K, g)
    assert t["bm"] > 0 and t["bn"] > 0 and t["bk"] == 128
    tiles = -(-M // t["bm"]) * -(-N // t["bn"])
    assert t["grid"] == tiles * t["ksplit"] or t["grid"] == tiles
    with pytest.raises(ValueError):
        dg.dg_query_tile(M, N, K + 1, g)


def test_python_binding_rejects_bad_tensors(dg):
    import torch

    a = torch.zeros((4, 128), dtype=torch.uint8)
    with pytest.raises(ValueError):
        dg.dg_gemm_fp8_nt(a, a, torch.ones(1, 1), torch.ones(1, 1))  # CPU tensors


# Host-side tile choice for the five workloads and shapes between them: M up
# to 128 streams; larger M takes the entry with the least estimated time.
@pytest.mark.parametrize("M,N,K,g,cls", [
    (256, 256, 256, 128, (32, 32, 1)),        # 64 tiles of 32x32
    (250, 1000, 2048, 128, (32, 32, 1)),      # few tiles, M > 128: the 32x32 streaming tiles
    (128, 7168, 2048, 64, (64, 64, 1)),       # M <= 128 with 896 tiles of 32x32: 224 of 64x64 win
    (128, 28672, 2048, 128, (128, 128, 1)),
    (600, 1000, 2048, 64, (64, 64, 1)),
    (777, 3333, 2048, 128, (128, 128, 1)),
    (1536, 7168, 2048, 128, (256, 256, 1)),   # 168 tiles of 256x256 beat 672 of 128x128
    (64, 4096, 7168, 128, (32, 32, 1)),       # small M, 256 streaming tiles
    (64, 512, 7168, 128, (32, 32, 1)),        # small M, few tiles: still 32x32 over the whole K (no workspace)
    (8, 300, 2048, 128, (32, 32, 1)),
    (4096, 7168, 2048, 128, (256, 256, 1)),   # 448 tiles of 256x256 (1.75 rounds) over 512 of 256x128
    (8192, 8192, 8192, 128, (256, 256, 1)),   # 1024 tiles of 256x256
    (2000, 4000, 16384, 64, (256, 128, 1)),   # 256 tiles of 256x128 vs 128 of 256x256
    (8192, 8192, 8192, 256, (256, 256, 1)),   # g = 256 runs the 128-segment kernels
    (64, 4096, 7168, 256, (32, 32, 1)),
])
def test_query_tile_choice(dg, M, N, K, g, cls):
    t = dg.dg_query_tile(M, N, K, g)
    assert (t["bm"], t["bn"], t["ksplit"]) == cls, t
    assert t["workspace_bytes"] == 0


# dg_gemm_fp8_ws's plan: K of at least 16384 (128 steps) that the 64x64
# tiles split at least 8 ways (any layout, any M) (round(256 / tiles), at
# most 16, at least 4 steps each) splits K over workgroups; everything else is
# the plan without a workspace, which needs no workspace.
@pytest.mark.parametrize("M,N,K,g,layout,cls", [
    (64, 512, 7168, 128, 0, (32, 32, 1)),      # K below 16384: streams, workspace or not
    (8, 300, 2048, 128, 0, (32, 32, 1)),
    (64, 512, 8192, 128, 0, (32, 32, 1)),      # 64 steps: streams
    (64, 512, 16384, 128, 0, (64, 64, 16)),    # 128 steps: 8 tiles, 32 splits capped at 16
    (64, 512, 24576, 128, 0, (64, 64, 16)),    # 8 tiles: 32 splits capped at 16
    (8, 256, 32768, 128, 0, (64, 64, 16)),     # 4 tiles: 64 capped at 16
    (64, 2048, 32768, 128, 1, (64, 64, 8)),    # B stored [K,N]: 32 tiles x 8 splits
    (64, 1024, 24576, 128, 3, (64, 64, 16)),   # 16 tiles x 16
    (96, 528, 24576, 256, 2, (64, 64, 14)),    # 18 tiles x 14 (g = 256 runs 128-segment steps)
    (128, 1024, 65536, 64, 0, (64, 64, 8)),    # g = 64: 32 tiles x 8
    (8, 4096, 32768, 128, 0, (32, 32, 1)),     # 64 tiles would give 4 splits: streams
    (256, 512, 32768, 128, 2, (64, 64, 8)),    # larger M, 32 tiles: 8 splits
    (2048, 64, 65536, 64, 0, (64, 64, 8)),
    (256, 1024, 32768, 128, 0, (32, 32, 1)),   # 64 tiles: 4 splits, the plan without a workspace
    (64, 4096, 32768, 128, 2, (32, 32, 1)),    # the same, A stored [K,M]
    (64, 4096, 7168, 128, 0, (32, 32, 1)),
    (8192, 8192, 8192, 128, 0, (256, 256, 1)),
])
def test_query_tile_ws_choice(dg, M, N, K, g, layout, cls):
    t = dg.dg_query_tile(M, N, K, g, layout, workspace=True)
    assert (t["bm"], t["bn"], t["ksplit"]) == cls, t
    tiles = -(-M // t["bm"]) * -(-N // t["bn"])
    assert t["grid"] == tiles * t["ksplit"]
    if t["ksplit"] == 1:
        assert t["workspace_bytes"] == 0
        assert t == dg.dg_query_tile(M, N, K, g, layout)
    else:
        # the FP32 partial tiles
        assert t["workspace_bytes"] == 4 * tiles * t["ksplit"] * 64 * 64


@pytest.mark.parametrize("M,N,K,g,layout,ksplit", [(64, 512, 7168, 128, 0, 14), (8, 300, 2048, 128, 3, 4),
                                                   (97, 531, 1088, 64, 1, 2), (64, 4096, 7168, 128, 2, 4)])
def test_forced_split_plan(dg, M, N, K, g, layout, ksplit):
    # DG_FORCE_TILE, read at every call: the split class on any shape, split
    # with a workspace, one split without; unset again, the plan is back
    from tests._common import forced_split

    free = dg.dg_query_tile(M, N, K, g, layout, workspace=True)
    with forced_split(g):
        t = dg.dg_query_tile(M, N, K, g, layout, workspace=True)
        assert (t["bm"], t["bn"], t["ksplit"]) == (64, 64, ksplit), t
        t1 = dg.dg_query_tile(M, N, K, g, layout)
        assert (t1["bm"], t1["bn"], t1["ksplit"], t1["workspace_bytes"]) == (64, 64, 1, 0), t1
    assert dg.dg_query_tile(M, N, K, g, layout, workspace=True) == free


# Fake addresses 2^40 apart for the workspace call, so that only the
# overlap a case plants can trigger the overlap rule.
WA, WB, WSA, WSB, WOUT, WS = (i << 40 for i in range(1, 7))


def _ws_call(dg, ws=WS, ws_bytes=4 << 20, M=64, N=512, K=32768, g=128, layout=0, sa_rows=None, out=WOUT, a=WA):
    return dg.lib.dg_gemm_fp8_ws(a, WB, WSA, WSB, out, M, N, K, g, layout, g if sa_rows is None else sa_rows, 0, 0,
                                 None, 0, ws, ws_bytes, None)


def test_ws_fake_addresses_do_not_overlap(dg):
    # the baseline case passes every argument check; it would then need a GPU,
    # so only its query is made here
    need = dg.dg_query_tile(64, 512, 32768, 128, 0, workspace=True)["workspace_bytes"]
    assert 0 < need <= 4 << 20
    assert max(64 * 32768, 512 * 32768, 2 * 64 * 512, 4 << 20) < 1 << 40


@pytest.mark.parametrize("kw,want", [
    (dict(ws=None, ws_bytes=4096), "DG_EINVAL"),            # a size without a buffer
    (dict(ws_bytes=0), "DG_EINVAL"),                        # a buffer without a size
    (dict(ws_bytes=-256), "DG_EINVAL"),
    (dict(ws=WS + 16), "DG_EALIGN"),                        # 256-byte alignment
    (dict(ws_bytes=4096), "DG_EINVAL"),                     # smaller than the 64x512x32768 plan needs
    (dict(ws=WOUT - 0x1000), "DG_EINVAL"),                  # overlaps out
    (dict(ws=WA + 0x1000), "DG_EINVAL"),                    # overlaps a
    (dict(out=WS + (1 << 19)), "DG_EINVAL"),                # out inside the workspace
    (dict(a=WA + 8), "DG_EALIGN"),
])
def test_ws_rejects(dg, kw, want):
    assert _ws_call(dg, **kw) == getattr(dg, want)


# The output may overlap no input (the inputs may overlap each other): each
# case is rejected before any HIP call.
@pytest.mark.parametrize("kw", [dict(out=A + 0x1000), dict(out=B), dict(sa=OUT + 0x200), dict(sb=OUT + 0x1fff0),
                                dict(out=SB - 0x100)])
def test_output_overlapping_an_input(dg, kw):
    assert _call(dg, **kw) == dg.DG_EINVAL


def test_bias_overlapping_the_output(dg):
    assert dg.lib.dg_gemm_fp8_nt_epi(A, B, SA, SB, OUT, 256, 256, 256, 128, 0, 0, OUT + 0x100, 1, None) == dg.DG_EINVAL


@pytest.mark.parametrize("x,q,s", [(A, A + 0x100, SA), (A, B, B + 0x10), (A, B, A + 0xff00), (A, A, SA)])
def test_quantize_overlaps(dg, x, q, s):
    # x [64][256] FP32 is 64 KB from A, q 16 KB, the factors 2 x 2 (or 64 x 2 per row) FP32
    assert dg.lib.dg_quantize_fp8_blocks(x, 64, 256, 128, 0, q, s, None) == dg.DG_EINVAL
    assert dg.lib.dg_quantize_fp8_rows(x, 64, 256, 128, 0, q, s, None) == dg.DG_EINVAL

@pytest.mark.parametrize("in_type", [3, -1, 7])
def test_quantize_typed_rejects_unknown_input_kind(dg, in_type):
    for fn in (dg.lib.dg_quantize_fp8_blocks_typed, dg.lib.dg_quantize_fp8_rows_typed):
        assert fn(A, in_type, 64, 256, 128, 0, B, SA, None) == dg.DG_EINVAL


@pytest.mark.parametrize("fmt,g,cols", [(2, 128, 256), (1, 96, 192), (0, 256, 384), (0, 128, 0)])
@pytest.mark.parametrize("in_type", [0, 1, 2])
def test_quantize_typed_einval(dg, in_type, fmt, g, cols):
    for fn in (dg.lib.dg_quantize_fp8_blocks_typed, dg.lib.dg_quantize_fp8_rows_typed):
        assert fn(A, in_type, 64, cols, g, fmt, B, SA, None) == dg.DG_EINVAL


def test_quantize_typed_alignment(dg):
    # x 16-byte aligned always; q 8-byte aligned for 16-bit input (a lane
    # writes eight codes), 4-byte for FP32
    for fn in (dg.lib.dg_quantize_fp8_blocks_typed, dg.lib.dg_quantize_fp8_rows_typed):
        for in_type in (1, 2):
            assert fn(A, in_type, 64, 256, 128, 0, B + 4, SA, None) == dg.DG_EALIGN
            assert fn(A + 8, in_type, 64, 256, 128, 0, B, SA, None) == dg.DG_EALIGN
        assert fn(A + 8, 0, 64, 256, 128, 0, B, SA, None) == dg.DG_EALIGN
        # FP32 input with q 4-byte aligned passes every argument check; what
        # follows is the device check (no GPU here) or a launch
        assert fn(A, 0, 64, 256, 128, 0, B + 4, SA, None) not in (dg.DG_EALIGN, dg.DG_EINVAL)


@pytest.mark.parametrize("in_type,q_off,overlaps", [(1, 0x7F00, True), (1, 0x8000, False), (2, 0x7FF8, True),
                                                    (2, 0x8000, False), (0, 0x8000, True), (0, 0x10000, False)])
def test_quantize_typed_overlap_counts_element_bytes(dg, in_type, q_off, overlaps):
    # x [64][256] is 32 KB of 16-bit elements, 64 KB of FP32; q is 16 KB
    rc = dg.lib.dg_quantize_fp8_blocks_typed(A, in_type, 64, 256, 128, 0, A + q_off, SB, None)
    assert (rc == dg.DG_EINVAL) == overlaps


def test_quantize_scale_count_cap(dg):
    """More than 2^31 - 1 scale factors is rejected before any device work.
    rows = 2^24 - 256 with 129 segments per row is 2,164,227,840 factors, and
    2^24 - 256 square in 64 x 64 blocks is 262,140^2. The fake addresses sit
    2^52 apart, beyond the 1.13e15 bytes of the largest x, so no overlap rule
    applies."""
    rows, g = (1 << 24) - 256, 64
    x, q, s = 1 << 52, 1 << 53, 1 << 54
    assert 4 * rows * rows < (1 << 52)
    assert dg.lib.dg_quantize_fp8_rows(x, rows, 129 * g, g, 0, q, s, None) == dg.DG_EINVAL
    assert dg.lib.dg_quantize_fp8_blocks(x, rows, rows, g, 0, q, s, None) == dg.DG_EINVAL
    for in_type in (0, 1, 2):
        assert dg.lib.dg_quantize_fp8_rows_typed(x, in_type, rows, 129 * g, g, 0, q, s, None) == dg.DG_EINVAL
        assert dg.lib.dg_quantize_fp8_blocks_typed(x, in_type, rows, rows, g, 0, q, s, None) == dg.DG_EINVAL


def test_noalloc_scratch_limit(dg):
    # the fixed scratch is 4 MiB; a plan needing more is refused before any HIP call
    assert dg.dg_noalloc_scratch_bytes() == 4 << 20
    M, N, K, g = 128, 1088, 32768, 128  # 34 tiles of 64x64 x 8 splits: 4.25 MiB of partials
    need = dg.dg_query_tile(M, N, K, g, workspace=True)["workspace_bytes"]
    assert need > dg.dg_noalloc_scratch_bytes()
    assert dg.lib.dg_gemm_fp8_noalloc(WA, WB, WSA, WSB, WOUT, M, N, K, g, 0, g, 0, 0, None, 0, None) == dg.DG_ESCRATCH
    # argument errors still come first
    assert dg.lib.dg_gemm_fp8_noalloc(0, WB, WSA, WSB, WOUT, M, N, K, g, 0, g, 0, 0, None, 0, None) == dg.DG_EINVAL


def test_tile_choice_is_the_same_for_every_layout(dg):
    """Every layout runs NT's plan (so every layout returns NT's bits), with
    and without a workspace, over a grid of shapes across all classes."""
    import itertools

    for M, N, K, g in itertools.product((1, 33, 128, 250, 777, 2000, 4096), (17, 1000, 4096, 28672),
                                        (256, 2048, 16384), (64, 128, 256)):
        if K % g:
            continue
        for ws in (False, True):
            nt = dg.dg_query_tile(M, N, K, g, 0, workspace=ws)
            for layout in (1, 2, 3):
                assert dg.dg_query_tile(M, N, K, g, layout, workspace=ws) == nt, (M, N, K, g, layout, ws)


def test_workspace_plans_stay_within_their_cap(dg):
    # a split plan's partials never exceed 16 MB, its splits 16, and every
    # split keeps at least 4 of the 128-byte K steps
    import itertools

    for M, N, K in itertools.product((1, 64, 128), (64, 1000, 4096, 8192), (16384, 65536, 1 << 20)):
        t = dg.dg_query_tile(M, N, K, 128, workspace=True)
        if t["ksplit"] > 1:
            assert t["workspace_bytes"] <= 16 << 20 and 8 <= t["ksplit"] <= 16
            assert K // 128 // t["ksplit"] >= 4

