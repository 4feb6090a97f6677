"""CPU oracle for the block-scaled FP8 GEMM (numpy front end over ``dgo.cpp``).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library never
imports, links or calls it, and it imports nothing from the HIP library.

The arithmetic lives in ``dgo.cpp``; its header states what each function
computes and which passage of the pages it follows:

* ``e4m3_decode`` / ``e4m3_encode``: OCP E4M3FN codec (the pages: "4 exponent
  bits, 3 mantissa bits"; input type torch.float8_e4m3fn, DeepGEMM实战 §4.2).
* ``quantize_blocks``: per g x g block, scale = amax/448 (FP32), codes =
  E4M3_RNE_SAT(x / scale) (DeepGEMM实战 §2.2, §4.4, §5.2).
* ``gemm_ref``: ref[i,j] = sum_kb sa[i/g,kb]*sb[j/g,kb] * P[i,j,kb] with the
  exact FP64 segment partials P (DeepGEMM实战 §2.2, §3.2, §3.3, §4.2).
* ``epilogue``: y = act(ref + bias[j]) in FP64, act none / ReLU / GELU (erf
  form) (the template article §2.3, §6: bias add, ReLU, GELU before the
  write-back).
* ``e5m2_decode`` / ``e5m2_encode``, ``quantize_blocks_fmt``, ``gemm_ref_fmt``:
  the same with E5M2 operands (DeepGEMM实战 §2.2 names E4M3 and E5M2 as the
  input formats; OCP E5M2 as torch.float8_e5m2 implements it), and any block
  granularity g (§3.1: 64, 128 and 256).
* ``gemm_ref_layout``: the reference GEMM with A stored [M,K] or [K,M] and B
  stored [N,K] or [K,N] (DeepGEMM实战 §3.3: either operand may be stored
  transposed); layout codes NT 0, NN 1, TT 2, TN 3.
* ``quantize_rows_fmt``, ``gemm_ref_rowa``: per-row A scales, one factor per
  row and g-wide K segment (1 x g blocks), B keeping its g x g blocks (the
  template article §3.4: per-tensor or per-channel factors, per channel the
  usual choice).

* ``bf16_decode``, ``f16_decode``, ``quantize_blocks_16``, ``quantize_rows_16``:
  the quantisers on BF16 or FP16 input (DeepGEMM实战 §4.4: the weights and
  activations to quantise come in FP16 or BF16): each input is decoded from
  its bit fields to its exact value (FP32 holds every finite one exactly) and
  the block rule above then applies unchanged.

Parity status: every function above is pinned by the CPU tests
(``tests/test_oracle_*.py``) against torch's float8 cast, brute force, exact
rational arithmetic, numpy's float64 matmul, closed forms and invariants.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dgo.cpp")
_LIB = os.path.join(_HERE, "libdgo.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``dgo.cpp`` into ``libdgo.so`` with plain g++ (no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.dgo_e4m3_decode.restype = ctypes.c_double
    lib.dgo_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.dgo_e4m3_encode.restype = ctypes.c_uint8
    lib.dgo_e4m3_encode.argtypes = [ctypes.c_float]
    lib.dgo_e4m3_decode_n.restype = None
    lib.dgo_e4m3_decode_n.argtypes = [u8p, i64, f64p]
    lib.dgo_e4m3_encode_n.restype = None
    lib.dgo_e4m3_encode_n.argtypes = [f32p, i64, u8p]
    lib.dgo_quantize_blocks.restype = ctypes.c_int
    lib.dgo_quantize_blocks.argtypes = [f32p, i64, i64, ctypes.c_int, u8p, f32p, ctypes.c_int]
    lib.dgo_segment_partials.restype = None
    lib.dgo_segment_partials.argtypes = [u8p, u8p, i64, ctypes.c_int, f64p]
    lib.dgo_gemm_ref.restype = ctypes.c_int
    lib.dgo_gemm_ref.argtypes = [u8p, u8p, f32p, f32p, i64, i64, i64, ctypes.c_int,
                                 i64p, i64, i64p, i64, f64p, ctypes.c_int]
    lib.dgo_e5m2_decode.restype = ctypes.c_double
    lib.dgo_e5m2_decode.argtypes = [ctypes.c_uint8]
    lib.dgo_e5m2_encode.restype = ctypes.c_uint8
    lib.dgo_e5m2_encode.argtypes = [ctypes.c_float]
    lib.dgo_e5m2_decode_n.restype = None
    lib.dgo_e5m2_decode_n.argtypes = [u8p, i64, f64p]
    lib.dgo_e5m2_encode_n.restype = None
    lib.dgo_e5m2_encode_n.argtypes = [f32p, i64, u8p]
    lib.dgo_quantize_blocks_fmt.restype = ctypes.c_int
    lib.dgo_quantize_blocks_fmt.argtypes = [f32p, i64, i64, ctypes.c_int, ctypes.c_int, u8p, f32p, ctypes.c_int]
    lib.dgo_gemm_ref_fmt.restype = ctypes.c_int
    lib.dgo_gemm_ref_fmt.argtypes = [u8p, u8p, f32p, f32p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, i64p, i64, i64p, i64, f64p, ctypes.c_int]
    lib.dgo_quantize_rows_fmt.restype = ctypes.c_int
    lib.dgo_quantize_rows_fmt.argtypes = [f32p, i64, i64, ctypes.c_int, ctypes.c_int, u8p, f32p, ctypes.c_int]
    lib.dgo_gemm_ref_rowa.restype = ctypes.c_int
    lib.dgo_gemm_ref_rowa.argtypes = [u8p, u8p, f32p, f32p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, i64p, i64, i64p, i64, f64p, ctypes.c_int]
    lib.dgo_gemm_ref_layout.restype = ctypes.c_int
    lib.dgo_gemm_ref_layout.argtypes = [u8p, u8p, f32p, f32p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, i64p, i64, i64p, i64, f64p, ctypes.c_int]
    lib.dgo_epilogue.restype = ctypes.c_int
    lib.dgo_epilogue.argtypes = [f64p, i64, i64, i64p, f32p, ctypes.c_int]
    u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.dgo_bf16_decode.restype = ctypes.c_double
    lib.dgo_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.dgo_f16_decode.restype = ctypes.c_double
    lib.dgo_f16_decode.argtypes = [ctypes.c_uint16]
    lib.dgo_decode16_n.restype = ctypes.c_int
    lib.dgo_decode16_n.argtypes = [u16p, i64, ctypes.c_int, f32p]
    lib.dgo_hardware_threads.restype = ctypes.c_int
    lib.dgo_hardware_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(arr: np.ndarray, ctype):
    return arr.ctypes.data_as(ctypes.POINTER(ctype))


# CPU share of one GPU on the hosts this runs on: worker pools stay within it
# whatever the host's hardware thread count.
CPU_SHARE = 16


def host_threads() -> int:
    """std::thread::hardware_concurrency() of this host."""
    return max(1, _load().dgo_hardware_threads())


def cpu_quota() -> int | None:
    """CPUs this process may use: its affinity mask, capped by a cgroup v2 cpu.max quota when one is set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            q = max(1, -(-int(quota) // int(period)))
            n = q if n is None else min(n, q)
    except (OSError, ValueError):
        pass
    return n


def default_threads() -> int:
    """Host threads the oracle uses: the hardware threads, within the process's
    CPU quota and the CPU share of one GPU (CPU_SHARE)."""
    n = min(host_threads(), CPU_SHARE)
    q = cpu_quota()
    return max(1, min(n, q) if q else n)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN codes (uint8, any shape) -> float64 values (NaN for 0x7F/0xFF)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().dgo_e4m3_decode_n(_ptr(c, ctypes.c_uint8), c.size, _ptr(out, ctypes.c_double))
    return out


def e4m3_encode(y) -> np.ndarray:
    """float32 values (any shape) -> E4M3FN codes, RNE, saturating at +-448."""
    v = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().dgo_e4m3_encode_n(_ptr(v, ctypes.c_float), v.size, _ptr(out, ctypes.c_uint8))
    return out


def quantize_blocks(x, g: int, nthreads: int | None = None):
    """x [rows, cols] float32 -> (codes uint8 [rows, cols], scales float32 [ceil(rows/g), cols/g])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % g:
        raise ValueError("cols must be a multiple of g")
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(((rows + g - 1) // g, cols // g), dtype=np.float32)
    rc = _load().dgo_quantize_blocks(_ptr(x, ctypes.c_float), rows, cols, g, _ptr(q, ctypes.c_uint8),
                                     _ptr(s, ctypes.c_float), nthreads or default_threads())
    if rc != 0:
        raise ValueError("dgo_quantize_blocks rejected its arguments")
    return q, s


def segment_partials(a_row, b_row, g: int) -> np.ndarray:
    """Exact FP64 segment partials P[kb] for one output element."""
    a_row = np.ascontiguousarray(a_row, dtype=np.uint8)
    b_row = np.ascontiguousarray(b_row, dtype=np.uint8)
    K = a_row.size
    P = np.empty(K // g, dtype=np.float64)
    _load().dgo_segment_partials(_ptr(a_row, ctypes.c_uint8), _ptr(b_row, ctypes.c_uint8), K, g,
                                 _ptr(P, ctypes.c_double))
    return P


def gemm_ref(a8, b8, sa, sb, g: int, rows=None, cols=None, nthreads: int | None = None) -> np.ndarray:
    """FP64 reference of C = A*B^T with block scales, on rows x cols of the output.

    a8 [M,K] uint8, b8 [N,K] uint8, sa [ceil(M/g), K/g] float32, sb [ceil(N/g), K/g] float32.
    rows / cols: optional index arrays; the result has shape [len(rows), len(cols)].
    """
    a8 = np.ascontiguousarray(a8, dtype=np.uint8)
    b8 = np.ascontiguousarray(b8, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    M, K = a8.shape
    N, K2 = b8.shape
    if K2 != K or K % g:
        raise ValueError("bad K")
    if sa.shape != ((M + g - 1) // g, K // g) or sb.shape != ((N + g - 1) // g, K // g):
        raise ValueError("bad scale shapes")
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    out = np.empty((nr, nc), dtype=np.float64)
    rc = _load().dgo_gemm_ref(
        _ptr(a8, ctypes.c_uint8), _ptr(b8, ctypes.c_uint8), _ptr(sa, ctypes.c_float),
        _ptr(sb, ctypes.c_float), M, N, K, g,
        None if r is None else _ptr(r, ctypes.c_int64), nr,
        None if c is None else _ptr(c, ctypes.c_int64), nc,
        _ptr(out, ctypes.c_double), nthreads or default_threads())
    if rc != 0:
        raise ValueError("dgo_gemm_ref rejected its arguments")
    return out



# Operand formats: 0 = E4M3FN, 1 = E5M2.
E4M3, E5M2 = 0, 1


def e5m2_decode(codes) -> np.ndarray:
    """E5M2 codes (uint8, any shape) -> float64 values (+-inf for 0x7C/0xFC, NaN above)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().dgo_e5m2_decode_n(_ptr(c, ctypes.c_uint8), c.size, _ptr(out, ctypes.c_double))
    return out


def e5m2_encode(y) -> np.ndarray:
    """float32 values (any shape) -> E5M2 codes, RNE, saturating at +-57344."""
    v = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().dgo_e5m2_encode_n(_ptr(v, ctypes.c_float), v.size, _ptr(out, ctypes.c_uint8))
    return out


def quantize_blocks_fmt(x, g: int, fmt: int, nthreads: int | None = None):
    """quantize_blocks for either format: scale = amax / (448 or 57344)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % g:
        raise ValueError("cols must be a multiple of g")
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(((rows + g - 1) // g, cols // g), dtype=np.float32)
    rc = _load().dgo_quantize_blocks_fmt(_ptr(x, ctypes.c_float), rows, cols, g, fmt, _ptr(q, ctypes.c_uint8),
                                         _ptr(s, ctypes.c_float), nthreads or default_threads())
    if rc != 0:
        raise ValueError("dgo_quantize_blocks_fmt rejected its arguments")
    return q, s


def gemm_ref_fmt(a8, b8, sa, sb, g: int, fmt_a: int, fmt_b: int, rows=None, cols=None,
                 nthreads: int | None = None) -> np.ndarray:
    """gemm_ref with the operands' formats given (0 = E4M3, 1 = E5M2)."""
    a8 = np.ascontiguousarray(a8, dtype=np.uint8)
    b8 = np.ascontiguousarray(b8, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    M, K = a8.shape
    N, K2 = b8.shape
    if K2 != K or K % g:
        raise ValueError("bad K")
    if sa.shape != ((M + g - 1) // g, K // g) or sb.shape != ((N + g - 1) // g, K // g):
        raise ValueError("bad scale shapes")
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    out = np.empty((nr, nc), dtype=np.float64)
    rc = _load().dgo_gemm_ref_fmt(
        _ptr(a8, ctypes.c_uint8), _ptr(b8, ctypes.c_uint8), _ptr(sa, ctypes.c_float),
        _ptr(sb, ctypes.c_float), M, N, K, g, fmt_a, fmt_b,
        None if r is None else _ptr(r, ctypes.c_int64), nr,
        None if c is None else _ptr(c, ctypes.c_int64), nc,
        _ptr(out, ctypes.c_double), nthreads or default_threads())
    if rc != 0:
        raise ValueError("dgo_gemm_ref_fmt rejected its arguments")
    return out


def quantize_rows_fmt(x, g: int, fmt: int = 0, nthreads: int | None = None):
    """1 x g quantisation: one factor per row and g-wide column segment; scales [rows, cols/g]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % g:
        raise ValueError("cols must be a multiple of g")
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows, cols // g), dtype=np.float32)
    rc = _load().dgo_quantize_rows_fmt(_ptr(x, ctypes.c_float), rows, cols, g, fmt, _ptr(q, ctypes.c_uint8),
                                       _ptr(s, ctypes.c_float), nthreads or default_threads())
    if rc != 0:
        raise ValueError("dgo_quantize_rows_fmt rejected its arguments")
    return q, s


def gemm_ref_rowa(a8, b8, sa, sb, g: int, fmt_a: int = 0, fmt_b: int = 0, rows=None, cols=None,
                  nthreads: int | None = None) -> np.ndarray:
    """Reference GEMM with per-row A scales: sa [M, K/g], sb [ceil(N/g), K/g]."""
    a8 = np.ascontiguousarray(a8, dtype=np.uint8)
    b8 = np.ascontiguousarray(b8, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    M, K = a8.shape
    N, K2 = b8.shape
    if K2 != K or K % g:
        raise ValueError("bad K")
    if sa.shape != (M, K // g) or sb.shape != ((N + g - 1) // g, K // g):
        raise ValueError("bad scale shapes")
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    out = np.empty((nr, nc), dtype=np.float64)
    rc = _load().dgo_gemm_ref_rowa(
        _ptr(a8, ctypes.c_uint8), _ptr(b8, ctypes.c_uint8), _ptr(sa, ctypes.c_float),
        _ptr(sb, ctypes.c_float), M, N, K, g, fmt_a, fmt_b,
        None if r is None else _ptr(r, ctypes.c_int64), nr,
        None if c is None else _ptr(c, ctypes.c_int64), nc,
        _ptr(out, ctypes.c_double), nthreads or default_threads())
    if rc != 0:
        raise ValueError("dgo_gemm_ref_rowa rejected its arguments")
    return out


# Operand layouts: bit 1 = A stored [K, M], bit 0 = B stored [K, N].
NT, NN, TT, TN = 0, 1, 2, 3


def gemm_ref_layout(a, b, sa, sb, g: int, layout: int, M: int, N: int, K: int, fmt_a: int = 0, fmt_b: int = 0,
                    rows=None, cols=None, nthreads: int | None = None) -> np.ndarray:
    """Reference GEMM with stored operands a ([M,K] or [K,M]) and b ([N,K] or [K,N]) per layout."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    want_a = (K, M) if layout & 2 else (M, K)
    want_b = (K, N) if layout & 1 else (N, K)
    if a.shape != want_a or b.shape != want_b or K % g:
        raise ValueError("operand shapes do not match the layout")
    if sa.shape != ((M + g - 1) // g, K // g) or sb.shape != ((N + g - 1) // g, K // g):
        raise ValueError("bad scale shapes")
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    out = np.empty((nr, nc), dtype=np.float64)
    rc = _load().dgo_gemm_ref_layout(
        _ptr(a, ctypes.c_uint8), _ptr(b, ctypes.c_uint8), _ptr(sa, ctypes.c_float), _ptr(sb, ctypes.c_float),
        M, N, K, g, layout, fmt_a, fmt_b,
        None if r is None else _ptr(r, ctypes.c_int64), nr,
        None if c is None else _ptr(c, ctypes.c_int64), nc,
        _ptr(out, ctypes.c_double), nthreads or default_threads())
    if rc != 0:
        raise ValueError("dgo_gemm_ref_layout rejected its arguments")
    return out


# Epilogue activations: 0 = none, 1 = ReLU, 2 = GELU (erf form).
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2


def epilogue(ref, bias=None, act: int = ACT_NONE, cols=None) -> np.ndarray:
    """act(ref + bias[cols]) in FP64 on a copy of ref [rows, len(cols)] (cols: output column indices)."""
    out = np.array(ref, dtype=np.float64, order="C", copy=True)
    nr, nc = out.shape
    c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    rc = _load().dgo_epilogue(_ptr(out, ctypes.c_double), nr, nc, None if c is None else _ptr(c, ctypes.c_int64),
                              None if b is None else _ptr(b, ctypes.c_float), act)
    if rc != 0:
        raise ValueError("dgo_epilogue rejected its arguments")
    return out


# 16-bit input kinds: 1 = BF16, 2 = FP16 (IEEE binary16).
IN_BF16 = 1
IN_F16 = 2


def decode16(bits, kind: int) -> np.ndarray:
    """16-bit patterns (uint16, any shape) of kind IN_BF16 or IN_F16 -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    if _load().dgo_decode16_n(_ptr(b, ctypes.c_uint16), b.size, kind, _ptr(out, ctypes.c_float)) != 0:
        raise ValueError("kind must be IN_BF16 or IN_F16")
    return out


def bf16_decode(bits) -> np.ndarray:
    """BF16 bit patterns -> float32 values."""
    return decode16(bits, IN_BF16)


def f16_decode(bits) -> np.ndarray:
    """FP16 bit patterns -> float32 values."""
    return decode16(bits, IN_F16)


def quantize_blocks_16(bits, kind: int, g: int, fmt: int = 0, nthreads: int | None = None):
    """g x g quantisation of a BF16 or FP16 matrix given as its bit patterns [rows, cols] (uint16)."""
    return quantize_blocks_fmt(decode16(bits, kind), g, fmt, nthreads)


def quantize_rows_16(bits, kind: int, g: int, fmt: int = 0, nthreads: int | None = None):
    """1 x g quantisation of a BF16 or FP16 matrix given as its bit patterns [rows, cols] (uint16)."""
    return quantize_rows_fmt(decode16(bits, kind), g, fmt, nthreads)
