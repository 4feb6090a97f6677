"""Block-scaled FP8 GEMM for AMD MI355X (gfx950): Python binding of libdg.so.

Argument marshalling only. Every step of the GEMM runs in the HIP kernels of
``libdg.so`` (C ABI in ``include/dg.h``); this module checks tensor dtypes,
shapes and devices, passes raw device pointers and the current HIP stream, and
turns status codes into exceptions. There is no fallback: if the library is
missing or fails to load, importing this package raises.

The operation (DeepGEMM实战 §2.2, §3.2, §4.2):
  out[i,j] = bf16( sum_kb sa[i/g,kb] * sb[j/g,kb] * sum_{k in kb} A[i,k] * B[j,k] )
with A [M,K], B [N,K] in E4M3FN or E5M2 (NT layout), FP32 scales per g x g
block (g = 64, 128 or 256) and FP32 accumulation within and across K segments.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime libdg.so binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")
# The same sources built with an extra full wait and workgroup barrier after
# every pipeline step (race check build; see load_library).
SYNC_LIB_PATH = os.path.join(_HERE, "libdg_sync.so")

DG_OK = 0
DG_EINVAL = -1
DG_EALIGN = -2
DG_EUNSUPPORTED = -3
DG_ELAUNCH = -4
DG_ESCRATCH = -5
DG_FMT_E4M3 = 0
DG_FMT_E5M2 = 1
DG_IN_F32 = 0
DG_IN_BF16 = 1
DG_IN_F16 = 2
DG_ACT_NONE = 0
DG_ACT_RELU = 1
DG_ACT_GELU = 2
DG_MAX_DIM = (1 << 24) - 256  # largest M, N or K (and quantiser rows, cols) the library accepts


class dg_tile_info(ctypes.Structure):
    _fields_ = [("kernel_id", ctypes.c_int), ("bm", ctypes.c_int), ("bn", ctypes.c_int),
                ("bk", ctypes.c_int), ("stages", ctypes.c_int), ("waves", ctypes.c_int),
                ("ksplit", ctypes.c_int), ("grid", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


def load_library(path: str):
    """Open a build of the C ABI at ``path`` (ctypes handle with every
    signature declared). The package itself uses libdg.so; the race check
    build libdg_sync.so is opened this way beside it (its own symbols, bound
    within itself) to compare the two builds' results."""
    if not os.path.exists(path):
        raise ImportError("%s is not built (run fp8_block_scaled_scales_amd.build.build()); "
                          "there is no non-HIP fallback" % os.path.basename(path))
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.dg_gemm_fp8_nt.restype = ctypes.c_int
    lib.dg_gemm_fp8_nt.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.dg_query_tile.restype = ctypes.c_int
    lib.dg_query_tile.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(dg_tile_info)]
    lib.dg_gemm_fp8_nt_fmt.restype = ctypes.c_int
    lib.dg_gemm_fp8_nt_fmt.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       vp]
    lib.dg_gemm_fp8_nt_epi.restype = ctypes.c_int
    lib.dg_gemm_fp8_nt_epi.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       vp, ctypes.c_int, vp]
    lib.dg_gemm_fp8_nt_ex.restype = ctypes.c_int
    lib.dg_gemm_fp8_nt_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, vp, ctypes.c_int, vp]
    lib.dg_gemm_fp8_layout.restype = ctypes.c_int
    lib.dg_gemm_fp8_layout.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, vp, ctypes.c_int, vp]
    lib.dg_query_tile_layout.restype = ctypes.c_int
    lib.dg_query_tile_layout.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(dg_tile_info)]
    lib.dg_query_tile_ws.restype = ctypes.c_int
    lib.dg_query_tile_ws.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(dg_tile_info)]
    lib.dg_gemm_fp8_ws.restype = ctypes.c_int
    lib.dg_gemm_fp8_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp, i64, vp]
    lib.dg_gemm_fp8_noalloc.restype = ctypes.c_int
    lib.dg_gemm_fp8_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp]
    lib.dg_noalloc_scratch_bytes.restype = ctypes.c_int64
    lib.dg_noalloc_scratch_bytes.argtypes = []
    lib.dg_quantize_fp8_rows.restype = ctypes.c_int
    lib.dg_quantize_fp8_rows.argtypes = [vp, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.dg_quantize_e4m3_blocks.restype = ctypes.c_int
    lib.dg_quantize_e4m3_blocks.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp, vp]
    lib.dg_quantize_fp8_blocks.restype = ctypes.c_int
    lib.dg_quantize_fp8_blocks.argtypes = [vp, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    for name in ("dg_quantize_fp8_blocks_typed", "dg_quantize_fp8_rows_typed"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, ctypes.c_int, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.dg_strerror.restype = ctypes.c_char_p
    lib.dg_strerror.argtypes = [ctypes.c_int]
    lib.dg_version.restype = ctypes.c_int
    lib.dg_version.argtypes = []
    return lib


_lib = load_library(LIB_PATH)
lib = _lib  # raw ctypes handle, for tests that exercise the C ABI directly


class DGError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, dg_strerror(code), code))
        self.code = code


class DGArgumentError(DGError, ValueError):
    pass


def _raise(code: int, where: str):
    if code in (DG_EINVAL, DG_EALIGN):
        raise DGArgumentError(code, where)
    raise DGError(code, where)


def dg_strerror(code: int) -> str:
    return _lib.dg_strerror(int(code)).decode()


def dg_version() -> int:
    return _lib.dg_version()


def dg_query_tile(M: int, N: int, K: int, gran: int = 128, layout: int = 0, workspace: bool = False) -> dict:
    """The tile-table plan of a call: dg_gemm_fp8_layout's (workspace=False) or dg_gemm_fp8_ws's."""
    info = dg_tile_info()
    fn = _lib.dg_query_tile_ws if workspace else _lib.dg_query_tile_layout
    rc = fn(M, N, K, gran, layout, ctypes.byref(info))
    if rc != DG_OK:
        _raise(rc, "dg_query_tile")
    return {name: getattr(info, name) for name, _ in dg_tile_info._fields_}


_FP8 = (torch.float8_e4m3fn, torch.uint8)
_FP8_OF = {DG_FMT_E4M3: (torch.float8_e4m3fn, torch.uint8), DG_FMT_E5M2: (torch.float8_e5m2, torch.uint8)}
_GRANS = (64, 128, 256)
_IN_OF = {torch.float32: DG_IN_F32, torch.bfloat16: DG_IN_BF16, torch.float16: DG_IN_F16}


def _check(t, name, dtypes, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _gemm(a, b, sa, sb, out, gran, fmt_a, fmt_b, stream, where, bias=None, act=DG_ACT_NONE, sa_rows=None):
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = a.shape
    N = b.shape[0]
    dev = a.device
    if gran not in _GRANS or K % gran:
        raise ValueError("gran must be 64, 128 or 256 and divide K")
    if fmt_a not in _FP8_OF or fmt_b not in _FP8_OF:
        raise ValueError("formats must be DG_FMT_E4M3 or DG_FMT_E5M2")
    sa_rows = gran if sa_rows is None else sa_rows
    if sa_rows not in (gran, 1):
        raise ValueError("sa_rows must be gran (g x g blocks) or 1 (per-row factors)")
    _check(a, "a", _FP8_OF[fmt_a], (M, K), dev)
    _check(b, "b", _FP8_OF[fmt_b], (N, K), dev)
    _check(sa, "sa", (torch.float32,), ((M + sa_rows - 1) // sa_rows, K // gran), dev)
    _check(sb, "sb", (torch.float32,), ((N + gran - 1) // gran, K // gran), dev)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _check(out, "out", (torch.bfloat16,), (M, N), dev)
    if bias is not None:
        _check(bias, "bias", (torch.float32,), (N,), dev)
    if act not in (DG_ACT_NONE, DG_ACT_RELU, DG_ACT_GELU):
        raise ValueError("act must be DG_ACT_NONE, DG_ACT_RELU or DG_ACT_GELU")
    if dev.type != "cuda":
        raise ValueError("a must be a GPU tensor")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        if where == "dg_gemm_fp8_nt_ex":
            rc = _lib.dg_gemm_fp8_nt_ex(a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(),
                                        M, N, K, gran, sa_rows, fmt_a, fmt_b,
                                        None if bias is None else bias.data_ptr(), act, s.cuda_stream)
        elif where == "dg_gemm_fp8_nt_epi":
            rc = _lib.dg_gemm_fp8_nt_epi(a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(),
                                         M, N, K, gran, fmt_a, fmt_b, None if bias is None else bias.data_ptr(),
                                         act, s.cuda_stream)
        elif fmt_a == DG_FMT_E4M3 and fmt_b == DG_FMT_E4M3 and where == "dg_gemm_fp8_nt":
            rc = _lib.dg_gemm_fp8_nt(a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(),
                                     M, N, K, gran, s.cuda_stream)
        else:
            rc = _lib.dg_gemm_fp8_nt_fmt(a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(),
                                         M, N, K, gran, fmt_a, fmt_b, s.cuda_stream)
    if rc != DG_OK:
        _raise(rc, where)
    return out


def dg_gemm_fp8_nt(a, b, sa, sb, out=None, gran: int = 128, stream=None):
    """out[M,N] (bf16) = A[M,K] * B[N,K]^T with gran x gran FP32 block scales.

    a: [M,K] float8_e4m3fn (or uint8 holding E4M3FN codes), b: [N,K] likewise,
    sa: [ceil(M/gran), K/gran] float32, sb: [ceil(N/gran), K/gran] float32,
    gran 64, 128 or 256, out: optional preallocated [M,N] bfloat16 (allocated
    when None). Enqueued on ``stream`` (a torch.cuda.Stream; default: the
    current stream).
    """
    return _gemm(a, b, sa, sb, out, gran, DG_FMT_E4M3, DG_FMT_E4M3, stream, "dg_gemm_fp8_nt")


def dg_gemm_fp8_nt_fmt(a, b, sa, sb, out=None, gran: int = 128, fmt_a: int = DG_FMT_E4M3,
                       fmt_b: int = DG_FMT_E4M3, stream=None):
    """dg_gemm_fp8_nt with each operand's FP8 format given (DG_FMT_E4M3 / DG_FMT_E5M2).

    An E5M2 operand is float8_e5m2 (or uint8 holding E5M2 codes).
    """
    return _gemm(a, b, sa, sb, out, gran, fmt_a, fmt_b, stream, "dg_gemm_fp8_nt_fmt")


def dg_gemm_fp8_nt_epi(a, b, sa, sb, out=None, gran: int = 128, fmt_a: int = DG_FMT_E4M3,
                       fmt_b: int = DG_FMT_E4M3, bias=None, act: int = DG_ACT_NONE, stream=None):
    """dg_gemm_fp8_nt_fmt with out = bf16(act(C + bias[None, :])) fused into the store.

    bias: optional [N] float32; act: DG_ACT_NONE, DG_ACT_RELU or DG_ACT_GELU (exact erf form).
    """
    return _gemm(a, b, sa, sb, out, gran, fmt_a, fmt_b, stream, "dg_gemm_fp8_nt_epi", bias, act)


def dg_gemm_fp8_nt_ex(a, b, sa, sb, out=None, gran: int = 128, sa_rows: int | None = None,
                      fmt_a: int = DG_FMT_E4M3, fmt_b: int = DG_FMT_E4M3, bias=None, act: int = DG_ACT_NONE,
                      stream=None):
    """dg_gemm_fp8_nt_epi with A's factor blocks chosen: sa_rows = gran (g x g, the default) or 1.

    With sa_rows = 1, sa is [M, K/gran] float32: one factor per row of A and K
    segment (per-row A scales); B keeps its g x g blocks.
    """
    return _gemm(a, b, sa, sb, out, gran, fmt_a, fmt_b, stream, "dg_gemm_fp8_nt_ex", bias, act, sa_rows)


# Operand layouts: bit 1 = A stored [K, M], bit 0 = B stored [K, N].
DG_LAYOUT_NT, DG_LAYOUT_NN, DG_LAYOUT_TT, DG_LAYOUT_TN = 0, 1, 2, 3


def dg_gemm_fp8_layout(a, b, sa, sb, out=None, gran: int = 128, layout: int = DG_LAYOUT_NT,
                       fmt_a: int = DG_FMT_E4M3, fmt_b: int = DG_FMT_E4M3, bias=None, act: int = DG_ACT_NONE,
                       stream=None):
    """dg_gemm_fp8_nt_epi with A stored [M,K] or [K,M] and B stored [N,K] or [K,N] per ``layout``.

    a: [M,K] (NT, NN) or [K,M] (TT, TN); b: [N,K] (NT, TT) or [K,N] (NN, TN); sa and
    sb keep their logical shapes [ceil(M/g), K/g] and [ceil(N/g), K/g]. M and N may
    be any length (ragged edges included) in every layout. Per-row A factors with
    a layout: dg_gemm_fp8_ws (workspace=None) takes both.
    """
    if layout not in (DG_LAYOUT_NT, DG_LAYOUT_NN, DG_LAYOUT_TT, DG_LAYOUT_TN):
        raise ValueError("layout must be DG_LAYOUT_NT, _NN, _TT or _TN")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    K, M = a.shape if layout & 2 else a.shape[::-1]
    N = b.shape[1] if layout & 1 else b.shape[0]
    dev = a.device
    if gran not in _GRANS or K % gran:
        raise ValueError("gran must be 64, 128 or 256 and divide K")
    if fmt_a not in _FP8_OF or fmt_b not in _FP8_OF:
        raise ValueError("formats must be DG_FMT_E4M3 or DG_FMT_E5M2")
    _check(a, "a", _FP8_OF[fmt_a], (K, M) if layout & 2 else (M, K), dev)
    _check(b, "b", _FP8_OF[fmt_b], (K, N) if layout & 1 else (N, K), dev)
    _check(sa, "sa", (torch.float32,), ((M + gran - 1) // gran, K // gran), dev)
    _check(sb, "sb", (torch.float32,), ((N + gran - 1) // gran, K // gran), dev)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _check(out, "out", (torch.bfloat16,), (M, N), dev)
    if bias is not None:
        _check(bias, "bias", (torch.float32,), (N,), dev)
    if act not in (DG_ACT_NONE, DG_ACT_RELU, DG_ACT_GELU):
        raise ValueError("act must be DG_ACT_NONE, DG_ACT_RELU or DG_ACT_GELU")
    if dev.type != "cuda":
        raise ValueError("a must be a GPU tensor")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = _lib.dg_gemm_fp8_layout(a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(),
                                     M, N, K, gran, layout, fmt_a, fmt_b, None if bias is None else bias.data_ptr(),
                                     act, s.cuda_stream)
    if rc != DG_OK:
        _raise(rc, "dg_gemm_fp8_layout")
    return out


def dg_workspace(M: int, N: int, K: int, gran: int = 128, layout: int = DG_LAYOUT_NT, device="cuda"):
    """A workspace for dg_gemm_fp8_ws of this shape (uint8 tensor), or None when its plan needs none."""
    n = dg_query_tile(M, N, K, gran, layout, workspace=True)["workspace_bytes"]
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _ws_args(a, b, sa, sb, out, gran, layout, sa_rows, fmt_a, fmt_b, bias, act):
    """Checks shared by dg_gemm_fp8_ws and dg_gemm_fp8_noalloc; returns (M, N, K, sa_rows, dev)."""
    if layout not in (DG_LAYOUT_NT, DG_LAYOUT_NN, DG_LAYOUT_TT, DG_LAYOUT_TN):
        raise ValueError("layout must be DG_LAYOUT_NT, _NN, _TT or _TN")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    K, M = a.shape if layout & 2 else a.shape[::-1]
    N = b.shape[1] if layout & 1 else b.shape[0]
    dev = a.device
    if gran not in _GRANS or K % gran:
        raise ValueError("gran must be 64, 128 or 256 and divide K")
    if fmt_a not in _FP8_OF or fmt_b not in _FP8_OF:
        raise ValueError("formats must be DG_FMT_E4M3 or DG_FMT_E5M2")
    sa_rows = gran if sa_rows is None else sa_rows
    if sa_rows not in (gran, 1):
        raise ValueError("sa_rows must be gran (g x g blocks) or 1 (per-row factors)")
    _check(a, "a", _FP8_OF[fmt_a], (K, M) if layout & 2 else (M, K), dev)
    _check(b, "b", _FP8_OF[fmt_b], (K, N) if layout & 1 else (N, K), dev)
    _check(sa, "sa", (torch.float32,), ((M + sa_rows - 1) // sa_rows, K // gran), dev)
    _check(sb, "sb", (torch.float32,), ((N + gran - 1) // gran, K // gran), dev)
    if out is not None:
        _check(out, "out", (torch.bfloat16,), (M, N), dev)
    if bias is not None:
        _check(bias, "bias", (torch.float32,), (N,), dev)
    if act not in (DG_ACT_NONE, DG_ACT_RELU, DG_ACT_GELU):
        raise ValueError("act must be DG_ACT_NONE, DG_ACT_RELU or DG_ACT_GELU")
    if dev.type != "cuda":
        raise ValueError("a must be a GPU tensor")
    return M, N, K, sa_rows, dev


def dg_gemm_fp8_ws(a, b, sa, sb, out=None, gran: int = 128, layout: int = DG_LAYOUT_NT, sa_rows: int | None = None,
                   fmt_a: int = DG_FMT_E4M3, fmt_b: int = DG_FMT_E4M3, bias=None, act: int = DG_ACT_NONE,
                   workspace=None, stream=None):
    """dg_gemm_fp8_layout (with dg_gemm_fp8_nt_ex's sa_rows) plus a caller-owned workspace.

    With a workspace (a contiguous uint8 GPU tensor of at least
    dg_query_tile(..., workspace=True)["workspace_bytes"] bytes, 256-byte
    aligned; see ``dg_workspace``) shapes with few output tiles and a long K
    (16384 and up, cut at least 8 ways) split K over several
    workgroups; every other shape runs what the call without a workspace
    runs. Concurrent calls need distinct workspaces.
    """
    M, N, K, sa_rows, dev = _ws_args(a, b, sa, sb, out, gran, layout, sa_rows, fmt_a, fmt_b, bias, act)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _check(workspace, "workspace", (torch.uint8,), (workspace.numel(),), dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = _lib.dg_gemm_fp8_ws(a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(),
                                 M, N, K, gran, layout, sa_rows, fmt_a, fmt_b,
                                 None if bias is None else bias.data_ptr(), act, ws_ptr, ws_bytes, s.cuda_stream)
    if rc != DG_OK:
        _raise(rc, "dg_gemm_fp8_ws")
    return out


def dg_gemm_fp8_noalloc(a, b, sa, sb, out, gran: int = 128, layout: int = DG_LAYOUT_NT, sa_rows: int | None = None,
                        fmt_a: int = DG_FMT_E4M3, fmt_b: int = DG_FMT_E4M3, bias=None, act: int = DG_ACT_NONE,
                        stream=None):
    """dg_gemm_fp8_ws with the library's fixed scratch array as the workspace: nothing is allocated.

    ``out`` must be given (this wrapper allocates nothing either). Calls that
    may overlap in time on one GPU race on the shared scratch; a plan that
    needs more than dg_noalloc_scratch_bytes() raises (DG_ESCRATCH).
    """
    if out is None:
        raise ValueError("dg_gemm_fp8_noalloc needs a preallocated out")
    M, N, K, sa_rows, dev = _ws_args(a, b, sa, sb, out, gran, layout, sa_rows, fmt_a, fmt_b, bias, act)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = _lib.dg_gemm_fp8_noalloc(a.data_ptr(), b.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(),
                                      M, N, K, gran, layout, sa_rows, fmt_a, fmt_b,
                                      None if bias is None else bias.data_ptr(), act, s.cuda_stream)
    if rc != DG_OK:
        _raise(rc, "dg_gemm_fp8_noalloc")
    return out


def dg_noalloc_scratch_bytes() -> int:
    return _lib.dg_noalloc_scratch_bytes()


def _quantize(x, gran, fmt, q, scales, stream, where):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor")
    rows, cols = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    if gran not in _GRANS or cols % gran:
        raise ValueError("gran must be 64, 128 or 256 and divide cols")
    if fmt not in _FP8_OF:
        raise ValueError("fmt must be DG_FMT_E4M3 or DG_FMT_E5M2")
    typed = where.endswith("_typed")
    _check(x, "x", tuple(_IN_OF) if typed else (torch.float32,), (rows, cols), dev)
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    brows = 1 if where.startswith("dg_quantize_fp8_rows") else gran  # rows per block
    if scales is None:
        scales = torch.empty(((rows + brows - 1) // brows, cols // gran), dtype=torch.float32, device=dev)
    _check(q, "q", _FP8_OF[fmt], (rows, cols), dev)
    _check(scales, "scales", (torch.float32,), ((rows + brows - 1) // brows, cols // gran), dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        if typed:
            rc = getattr(_lib, where)(x.data_ptr(), _IN_OF[x.dtype], rows, cols, gran, fmt, q.data_ptr(),
                                      scales.data_ptr(), s.cuda_stream)
        elif where == "dg_quantize_fp8_rows":
            rc = _lib.dg_quantize_fp8_rows(x.data_ptr(), rows, cols, gran, fmt, q.data_ptr(), scales.data_ptr(),
                                           s.cuda_stream)
        elif fmt == DG_FMT_E4M3 and where == "dg_quantize_e4m3_blocks":
            rc = _lib.dg_quantize_e4m3_blocks(x.data_ptr(), rows, cols, gran, q.data_ptr(), scales.data_ptr(),
                                              s.cuda_stream)
        else:
            rc = _lib.dg_quantize_fp8_blocks(x.data_ptr(), rows, cols, gran, fmt, q.data_ptr(), scales.data_ptr(),
                                             s.cuda_stream)
    if rc != DG_OK:
        _raise(rc, where)
    return q, scales


def dg_quantize_e4m3_blocks(x, gran: int = 128, q=None, scales=None, stream=None):
    """Block-quantise x [rows, cols] float32 on the GPU -> (q uint8 [rows, cols], scales float32).

    Per gran x gran block (gran 64, 128 or 256): scale = amax / 448 (1.0 for
    an all-zero block) and q = E4M3FN(x / scale), round to nearest even.
    ``scales`` has shape [ceil(rows/gran), cols/gran]. The codes come back as
    uint8 holding E4M3FN bytes (``q.view(torch.float8_e4m3fn)`` reinterprets
    them).
    """
    return _quantize(x, gran, DG_FMT_E4M3, q, scales, stream, "dg_quantize_e4m3_blocks")


def dg_quantize_fp8_blocks(x, gran: int = 128, fmt: int = DG_FMT_E4M3, q=None, scales=None, stream=None):
    """dg_quantize_e4m3_blocks for either format; E5M2 uses scale = amax / 57344."""
    return _quantize(x, gran, fmt, q, scales, stream, "dg_quantize_fp8_blocks")


def dg_quantize_fp8_rows(x, gran: int = 128, fmt: int = DG_FMT_E4M3, q=None, scales=None, stream=None):
    """1 x gran quantisation on the GPU: one factor per row and gran-wide segment, scales [rows, cols/gran]."""
    return _quantize(x, gran, fmt, q, scales, stream, "dg_quantize_fp8_rows")


def dg_quantize_fp8_blocks_typed(x, gran: int = 128, fmt: int = DG_FMT_E4M3, q=None, scales=None, stream=None):
    """dg_quantize_fp8_blocks on float32, bfloat16 or float16 x (the input kind is x's dtype).

    Each element is widened exactly to FP32 first, so a 16-bit x and its FP32
    copy give identical codes and scales.
    """
    return _quantize(x, gran, fmt, q, scales, stream, "dg_quantize_fp8_blocks_typed")


def dg_quantize_fp8_rows_typed(x, gran: int = 128, fmt: int = DG_FMT_E4M3, q=None, scales=None, stream=None):
    """dg_quantize_fp8_rows on float32, bfloat16 or float16 x (the input kind is x's dtype)."""
    return _quantize(x, gran, fmt, q, scales, stream, "dg_quantize_fp8_rows_typed")


__all__ = ["dg_gemm_fp8_nt", "dg_gemm_fp8_nt_fmt", "dg_gemm_fp8_nt_epi", "dg_gemm_fp8_nt_ex", "dg_gemm_fp8_layout",
           "dg_gemm_fp8_ws", "dg_workspace", "dg_gemm_fp8_noalloc", "dg_noalloc_scratch_bytes", "DG_ESCRATCH",
           "DG_LAYOUT_NT", "DG_LAYOUT_NN", "DG_LAYOUT_TT", "DG_LAYOUT_TN", "DG_ACT_NONE",
           "DG_ACT_RELU", "DG_ACT_GELU", "dg_quantize_e4m3_blocks", "dg_quantize_fp8_blocks", "dg_quantize_fp8_rows",
           "dg_quantize_fp8_blocks_typed", "dg_quantize_fp8_rows_typed", "DG_IN_F32", "DG_IN_BF16", "DG_IN_F16",
           "dg_query_tile", "dg_strerror", "dg_version", "DGError", "DGArgumentError", "DG_OK", "DG_EINVAL",
           "DG_EALIGN", "DG_EUNSUPPORTED", "DG_ELAUNCH", "DG_FMT_E4M3", "DG_FMT_E5M2", "DG_MAX_DIM", "LIB_PATH"]
