"""Python binding of the gfx950 ragged-M grouped GEMM library.

Argument marshalling only: every step of the computation runs in the HIP
library (``libmoe_ragged_grouped_amd.so``, built from ``csrc/``). PyTorch
supplies device memory and the stream. There is no fallback: if the library
is missing or a call fails, an exception is raised.

    C = grouped_gemm(A, B, offsets)            # A [M_cap,K] bf16, B [E,K,N] bf16,
                                               # offsets int32 [E+1], C [M_cap,N] fp32
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["grouped_gemm", "grouped_gemm_swiglu", "grouped_gemm_gather",
           "grouped_gemm_gather_combine", "grouped_gemm_fp8w", "grouped_gemm_fp8",
           "grouped_gemm_fp8_swiglu", "tile_schedule", "library_path", "load_library",
           "traced_grouped_gemm", "trace_library_path", "load_trace_library",
           "GroupedGemmError", "BM_CHOICES", "TILE_N", "MAX_EXPERTS", "SYMBOLS",
           "TRACE_SYMBOLS", "TRACE_WORKGROUPS", "TRACE_RECORD"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_ragged_grouped_amd.so")

BM_CHOICES = (16, 32, 64, 128, 256)
# narrowest tile width: sizes the host-side upper bound of the tile count
TILE_N = 256
MAX_EXPERTS = 1024
SYMBOLS = ("gg_grouped_gemm_bf16", "gg_grouped_gemm_bf16_bf16out", "gg_grouped_gemm_bf16_swiglu",
           "gg_grouped_gemm_bf16_gather", "gg_grouped_gemm_bf16_gather_combine",
           "gg_grouped_gemm_fp8w", "gg_grouped_gemm_fp8", "gg_grouped_gemm_fp8_bf16out",
           "gg_grouped_gemm_fp8_swiglu", "gg_tile_schedule", "gg_status_string")

# the tracing build (include/grouped_gemm_trace.h): a diagnostic library
_TRACE_LIB_PATH = os.path.join(_HERE, "libmoe_ragged_grouped_amd_trace.so")
TRACE_SYMBOLS = ("gg_trace_grouped_gemm_bf16", "gg_trace_clock_khz")
TRACE_WORKGROUPS = 1024
TRACE_RECORD = 8  # uint64 values per record

_lib = None
_trace_lib = None


class GroupedGemmError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise GroupedGemmError(
                "HIP library %s is not built; run `python -m moe_ragged_grouped_amd.build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.gg_grouped_gemm_bf16.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        lib.gg_grouped_gemm_bf16.restype = ctypes.c_int
        lib.gg_grouped_gemm_bf16_bf16out.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        lib.gg_grouped_gemm_bf16_bf16out.restype = ctypes.c_int
        lib.gg_grouped_gemm_bf16_swiglu.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        lib.gg_grouped_gemm_bf16_swiglu.restype = ctypes.c_int
        lib.gg_grouped_gemm_bf16_gather.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                    i32, vp]
        lib.gg_grouped_gemm_bf16_gather.restype = ctypes.c_int
        lib.gg_grouped_gemm_bf16_gather_combine.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32,
                                                            i32, i32, i32, i32, i32, vp]
        lib.gg_grouped_gemm_bf16_gather_combine.restype = ctypes.c_int
        lib.gg_grouped_gemm_fp8w.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        lib.gg_grouped_gemm_fp8w.restype = ctypes.c_int
        lib.gg_grouped_gemm_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        lib.gg_grouped_gemm_fp8.restype = ctypes.c_int
        lib.gg_grouped_gemm_fp8_bf16out.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                    i32, vp]
        lib.gg_grouped_gemm_fp8_bf16out.restype = ctypes.c_int
        lib.gg_grouped_gemm_fp8_swiglu.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                   i32, vp]
        lib.gg_grouped_gemm_fp8_swiglu.restype = ctypes.c_int
        lib.gg_tile_schedule.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, vp]
        lib.gg_tile_schedule.restype = ctypes.c_int
        lib.gg_status_string.argtypes = [ctypes.c_int]
        lib.gg_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().gg_status_string(status).decode()
        raise GroupedGemmError("%s: status %d (%s)" % (what, status, msg))


def _stream_handle(device, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _grouped_args(A, B, offsets):
    """Checks A bf16 [M_cap, K], B bf16 [E, K, N], offsets int32 [E+1] (device,
    contiguous); returns E, K, N, M_cap."""
    import torch
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if offsets.dtype != torch.int32:
        raise TypeError("offsets must be int32")
    if A.dim() != 2 or B.dim() != 3 or offsets.dim() != 1:
        raise ValueError("shapes: A [M_cap,K], B [E,K,N], offsets [E+1]")
    if not (A.is_cuda and B.is_cuda and offsets.is_cuda):
        raise ValueError("A, B and offsets must be device tensors")
    if not (A.is_contiguous() and B.is_contiguous() and offsets.is_contiguous()):
        raise ValueError("A, B and offsets must be contiguous")
    E, K, N = B.shape
    M_cap = A.shape[0]
    if A.shape[1] != K or offsets.shape[0] != E + 1:
        raise ValueError("shape mismatch: A %s, B %s, offsets %s" % (tuple(A.shape), tuple(B.shape),
                                                                      tuple(offsets.shape)))
    return E, K, N, M_cap


def grouped_gemm(A, B, offsets, out=None, bm: int = 0, stream=None, out_dtype=None):
    """C[off[e]:off[e+1]] = A[off[e]:off[e+1]] @ B[e] for every expert e, in one launch.

    A: bf16 [M_cap, K]; B: bf16 [E, K, N]; offsets: int32 [E+1] (device);
    out: optional fp32 or bf16 [M_cap, N] (out_dtype, default fp32, when out
    is not given); bm: 0 (per-expert choice on the device) or
    16/32/64/128/256. A bf16 ``out`` receives the fp32 result rounded to
    nearest even. Rows of ``out`` at or past offsets[E] are left as they
    were. Enqueued on ``stream`` (default: torch's current stream).
    """
    import torch
    lib = load_library()
    E, K, N, M_cap = _grouped_args(A, B, offsets)
    if out is None:
        dt = torch.float32 if out_dtype is None else out_dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
        out = torch.empty((M_cap, N), dtype=dt, device=A.device)
    elif (out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (M_cap, N)
          or not out.is_contiguous() or (out_dtype is not None and out.dtype != out_dtype)):
        raise ValueError("out must be a contiguous fp32 or bf16 [M_cap, N] tensor")
    fn = lib.gg_grouped_gemm_bf16 if out.dtype == torch.float32 else lib.gg_grouped_gemm_bf16_bf16out
    st = fn(A.data_ptr(), B.data_ptr(), offsets.data_ptr(), out.data_ptr(), E, K, N, M_cap, int(bm),
            _stream_handle(A.device, stream))
    _check(st, fn.__name__)
    return out


def grouped_gemm_swiglu(A, B, offsets, out=None, bm: int = 0, stream=None):
    """H[r, j] = silu(C[r, 2j]) * C[r, 2j+1] for C = the grouped product, in one launch.

    A, B, offsets, bm and stream as in grouped_gemm; B's columns hold the
    gate and up projections interleaved (column 2j gate j, column 2j+1 up j).
    out: optional bf16 [M_cap, N // 2]. The activation runs in fp32 in the
    kernel's epilogue and is rounded once to bf16. Rows at or past
    offsets[E] are left as they were.
    """
    import torch
    lib = load_library()
    E, K, N, M_cap = _grouped_args(A, B, offsets)
    if out is None:
        out = torch.empty((M_cap, N // 2), dtype=torch.bfloat16, device=A.device)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != (M_cap, N // 2)
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bf16 [M_cap, N // 2] tensor")
    st = lib.gg_grouped_gemm_bf16_swiglu(A.data_ptr(), B.data_ptr(), offsets.data_ptr(),
                                         out.data_ptr(), E, K, N, M_cap, int(bm),
                                         _stream_handle(A.device, stream))
    _check(st, "gg_grouped_gemm_bf16_swiglu")
    return out


def grouped_gemm_gather(X, src_rows, B, offsets, dst_rows=None, out=None, bm: int = 0,
                        stream=None):
    """The grouped product with rows gathered and scattered by index, in one launch.

    X: bf16 [n_src, K]; src_rows: int32 [M_cap] (device): grouped row r reads
    X[src_rows[r]] (rows of expert e are offsets[e]..offsets[e+1]-1);
    dst_rows: optional int32 [M_cap]: grouped row r is written to
    out[dst_rows[r]] (default: out[r]); B, offsets, bm, stream as in
    grouped_gemm; out: optional fp32 [M_cap, N]. Indices out of range read
    zeros (src) or are not written (dst).
    """
    import torch
    lib = load_library()
    if X.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("X and B must be bfloat16")
    if src_rows.dtype != torch.int32 or offsets.dtype != torch.int32 or (
            dst_rows is not None and dst_rows.dtype != torch.int32):
        raise TypeError("src_rows, dst_rows and offsets must be int32")
    if X.dim() != 2 or B.dim() != 3 or offsets.dim() != 1 or src_rows.dim() != 1:
        raise ValueError("shapes: X [n_src,K], src_rows [M_cap], B [E,K,N], offsets [E+1]")
    tensors = [X, B, offsets, src_rows] + ([dst_rows] if dst_rows is not None else [])
    if not all(t.is_cuda and t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous device tensors")
    E, K, N = B.shape
    n_src, M_cap = X.shape[0], src_rows.shape[0]
    if X.shape[1] != K or offsets.shape[0] != E + 1 or (
            dst_rows is not None and dst_rows.shape[0] != M_cap):
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M_cap, N), dtype=torch.float32, device=X.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M_cap, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [M_cap, N] tensor")
    st = lib.gg_grouped_gemm_bf16_gather(
        X.data_ptr(), n_src, src_rows.data_ptr(), B.data_ptr(), offsets.data_ptr(), out.data_ptr(),
        dst_rows.data_ptr() if dst_rows is not None else None, E, K, N, M_cap, int(bm),
        _stream_handle(X.device, stream))
    _check(st, "gg_grouped_gemm_bf16_gather")
    return out


def grouped_gemm_gather_combine(X, src_rows, B, offsets, dst_rows, weights, out=None,
                                n_dst=None, bm: int = 0, stream=None):
    """out[dst_rows[r]] += weights[r] * (X[src_rows[r]] @ B[e(r)]) for every routed row r, in one launch.

    X, src_rows, B, offsets, bm, stream as in grouped_gemm_gather; dst_rows
    int32 [M_cap] and weights fp32 [M_cap] (device) are required. out: fp32
    [n_dst, N], accumulated into (default: zeros with n_dst = n_src rows, the
    token rows). Destinations outside [0, n_dst) are skipped. The adds are
    fp32 atomics, so the rounding of each element's sum depends on the order
    the adds land in.
    """
    import torch
    lib = load_library()
    if X.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("X and B must be bfloat16")
    if (src_rows.dtype != torch.int32 or offsets.dtype != torch.int32
            or dst_rows.dtype != torch.int32):
        raise TypeError("src_rows, dst_rows and offsets must be int32")
    if weights.dtype != torch.float32:
        raise TypeError("weights must be float32")
    if (X.dim() != 2 or B.dim() != 3 or offsets.dim() != 1 or src_rows.dim() != 1
            or dst_rows.dim() != 1 or weights.dim() != 1):
        raise ValueError("shapes: X [n_src,K], src_rows/dst_rows/weights [M_cap], B [E,K,N], "
                         "offsets [E+1]")
    tensors = [X, B, offsets, src_rows, dst_rows, weights]
    if not all(t.is_cuda and t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous device tensors")
    E, K, N = B.shape
    n_src, M_cap = X.shape[0], src_rows.shape[0]
    if (X.shape[1] != K or offsets.shape[0] != E + 1 or dst_rows.shape[0] != M_cap
            or weights.shape[0] != M_cap):
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.zeros((n_src if n_dst is None else int(n_dst), N), dtype=torch.float32,
                          device=X.device)
    elif out.dtype != torch.float32 or out.dim() != 2 or out.shape[1] != N or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [n_dst, N] tensor")
    st = lib.gg_grouped_gemm_bf16_gather_combine(
        X.data_ptr(), n_src, src_rows.data_ptr(), B.data_ptr(), offsets.data_ptr(),
        dst_rows.data_ptr(), weights.data_ptr(), out.data_ptr(), out.shape[0], E, K, N, M_cap,
        int(bm), _stream_handle(X.device, stream))
    _check(st, "gg_grouped_gemm_bf16_gather_combine")
    return out


def grouped_gemm_fp8w(A, Bq, b_scale, offsets, out=None, bm: int = 0, stream=None):
    """The grouped product with fp8 (OCP E4M3) weights and per-column scales.

    A: bf16 [M_cap, K]; Bq: uint8 (or float8_e4m3fn) [E, K, N]; b_scale: fp32
    [E, N]; offsets: int32 [E+1]. out[r, n] = b_scale[e, n] * sum_k A[r, k] *
    Bq[e, k, n] for the rows r of expert e (fp32 [M_cap, N]).
    """
    import torch
    lib = load_library()
    if A.dtype != torch.bfloat16 or Bq.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("A must be bfloat16 and Bq uint8 / float8_e4m3fn")
    if b_scale.dtype != torch.float32 or offsets.dtype != torch.int32:
        raise TypeError("b_scale must be float32 and offsets int32")
    if A.dim() != 2 or Bq.dim() != 3 or b_scale.dim() != 2 or offsets.dim() != 1:
        raise ValueError("shapes: A [M_cap,K], Bq [E,K,N], b_scale [E,N], offsets [E+1]")
    if not all(t.is_cuda and t.is_contiguous() for t in (A, Bq, b_scale, offsets)):
        raise ValueError("all tensors must be contiguous device tensors")
    E, K, N = Bq.shape
    M_cap = A.shape[0]
    if A.shape[1] != K or tuple(b_scale.shape) != (E, N) or offsets.shape[0] != E + 1:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M_cap, N), dtype=torch.float32, device=A.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M_cap, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [M_cap, N] tensor")
    st = lib.gg_grouped_gemm_fp8w(A.data_ptr(), Bq.data_ptr(), b_scale.data_ptr(), offsets.data_ptr(),
                                  out.data_ptr(), E, K, N, M_cap, int(bm),
                                  _stream_handle(A.device, stream))
    _check(st, "gg_grouped_gemm_fp8w")
    return out


def grouped_gemm_fp8(Aq, a_scale, Bq, b_scale, offsets, out=None, bm: int = 0, stream=None,
                     out_dtype=None):
    """C = (a_scale * dec(Aq)) @ (dec(Bq[e]) * b_scale[e]) per expert, fp8 matrix cores.

    Aq: uint8 [M_cap, K] E4M3 codes; a_scale: fp32 [M_cap]; Bq: uint8
    [E, K, N] E4M3 codes; b_scale: fp32 [E, N]; offsets int32 [E+1]; out:
    optional fp32 or bf16 [M_cap, N] (out_dtype when out is not given,
    default fp32; bf16 is the fp32 result rounded to nearest even). K and N
    must be multiples of 16.
    """
    import torch
    lib = load_library()
    if Aq.dtype != torch.uint8 or Bq.dtype != torch.uint8:
        raise TypeError("Aq and Bq must be uint8 E4M3 codes")
    if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
        raise TypeError("a_scale and b_scale must be float32")
    if offsets.dtype != torch.int32:
        raise TypeError("offsets must be int32")
    if Aq.dim() != 2 or Bq.dim() != 3 or a_scale.dim() != 1 or b_scale.dim() != 2:
        raise ValueError("shapes: Aq [M_cap,K], a_scale [M_cap], Bq [E,K,N], b_scale [E,N]")
    tensors = [Aq, a_scale, Bq, b_scale, offsets]
    if not all(t.is_cuda and t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous device tensors")
    E, K, N = Bq.shape
    M_cap = Aq.shape[0]
    if (Aq.shape[1] != K or a_scale.shape[0] != M_cap or tuple(b_scale.shape) != (E, N)
            or offsets.shape[0] != E + 1):
        raise ValueError("shape mismatch")
    if out is None:
        dt = torch.float32 if out_dtype is None else out_dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
        out = torch.empty((M_cap, N), dtype=dt, device=Aq.device)
    elif (out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (M_cap, N)
          or not out.is_contiguous() or (out_dtype is not None and out.dtype != out_dtype)):
        raise ValueError("out must be a contiguous fp32 or bf16 [M_cap, N] tensor")
    fn = lib.gg_grouped_gemm_fp8 if out.dtype == torch.float32 else lib.gg_grouped_gemm_fp8_bf16out
    st = fn(Aq.data_ptr(), a_scale.data_ptr(), Bq.data_ptr(), b_scale.data_ptr(),
            offsets.data_ptr(), out.data_ptr(), E, K, N, M_cap, int(bm),
            _stream_handle(Aq.device, stream))
    _check(st, fn.__name__)
    return out


def grouped_gemm_fp8_swiglu(Aq, a_scale, Bq, b_scale, offsets, out=None, bm: int = 0,
                            stream=None):
    """H[r, j] = silu(C[r, 2j]) * C[r, 2j+1] for C = the fp8 x fp8 product.

    Arguments as in grouped_gemm_fp8; Bq's columns interleave gate (even) and
    up (odd); out: optional bf16 [M_cap, N // 2].
    """
    import torch
    lib = load_library()
    if Aq.dtype != torch.uint8 or Bq.dtype != torch.uint8:
        raise TypeError("Aq and Bq must be uint8 E4M3 codes")
    if a_scale.dtype != torch.float32 or b_scale.dtype != torch.float32:
        raise TypeError("a_scale and b_scale must be float32")
    if offsets.dtype != torch.int32:
        raise TypeError("offsets must be int32")
    tensors = [Aq, a_scale, Bq, b_scale, offsets]
    if not all(t.is_cuda and t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous device tensors")
    E, K, N = Bq.shape
    M_cap = Aq.shape[0]
    if (Aq.dim() != 2 or Aq.shape[1] != K or tuple(a_scale.shape) != (M_cap,)
            or tuple(b_scale.shape) != (E, N) or tuple(offsets.shape) != (E + 1,)):
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M_cap, N // 2), dtype=torch.bfloat16, device=Aq.device)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != (M_cap, N // 2)
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bf16 [M_cap, N // 2] tensor")
    st = lib.gg_grouped_gemm_fp8_swiglu(Aq.data_ptr(), a_scale.data_ptr(), Bq.data_ptr(),
                                        b_scale.data_ptr(), offsets.data_ptr(), out.data_ptr(),
                                        E, K, N, M_cap, int(bm), _stream_handle(Aq.device, stream))
    _check(st, "gg_grouped_gemm_fp8_swiglu")
    return out


def tile_schedule(offsets, N: int, M_cap: int, bm: int = 0, max_tiles: int = None, stream=None):
    """The device-built tile list: int32 tensor [n_tiles, 5] of (expert, row0, rows, col0, bm)."""
    import torch
    lib = load_library()
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.dim() != 1:
        raise TypeError("offsets must be a 1-D int32 device tensor")
    E = offsets.shape[0] - 1
    if max_tiles is None:
        hmin = bm if bm else BM_CHOICES[0]
        max_tiles = (M_cap // hmin + E) * (-(-N // TILE_N))
    tiles = torch.empty((max(max_tiles, 1), 5), dtype=torch.int32, device=offsets.device)
    n = torch.zeros(1, dtype=torch.int32, device=offsets.device)
    st = lib.gg_tile_schedule(offsets.data_ptr(), E, N, M_cap, int(bm), tiles.data_ptr(), n.data_ptr(),
                              int(max_tiles), _stream_handle(offsets.device, stream))
    _check(st, "gg_tile_schedule")
    count = int(n.item())
    return tiles[:min(count, max_tiles)], count


def trace_library_path() -> str:
    return _TRACE_LIB_PATH


def load_trace_library():
    """Load the tracing build (raises if it has not been built)."""
    global _trace_lib
    if _trace_lib is None:
        if not os.path.exists(_TRACE_LIB_PATH):
            raise GroupedGemmError(
                "HIP library %s is not built; run `python -m moe_ragged_grouped_amd.build`"
                % _TRACE_LIB_PATH)
        lib = ctypes.CDLL(_TRACE_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.gg_trace_grouped_gemm_bf16.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp,
                                                   i32, vp]
        lib.gg_trace_grouped_gemm_bf16.restype = ctypes.c_int
        lib.gg_trace_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int32)]
        lib.gg_trace_clock_khz.restype = ctypes.c_int
        lib.gg_status_string.argtypes = [ctypes.c_int]
        lib.gg_status_string.restype = ctypes.c_char_p
        _trace_lib = lib
    return _trace_lib


def traced_grouped_gemm(A, B, offsets, max_tiles: int, out=None, bm: int = 0, stream=None,
                        trace=None):
    """grouped_gemm (fp32 C) through the tracing build, with its timeline.

    Returns (C, trace, khz): trace is the uint64 record buffer of
    gg_trace_grouped_gemm_bf16 as an int64 device tensor
    [TRACE_WORKGROUPS + max_tiles, TRACE_RECORD], khz the rate of its
    counter. A trace tensor passed in is written as it is (records the launch
    does not write keep their values); otherwise a cleared one is allocated.
    """
    import torch
    lib = load_trace_library()
    E, K, N, M_cap = _grouped_args(A, B, offsets)
    if out is None:
        out = torch.empty((M_cap, N), dtype=torch.float32, device=A.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M_cap, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [M_cap, N] tensor")
    shape = (TRACE_WORKGROUPS + int(max_tiles), TRACE_RECORD)
    if trace is None:
        trace = torch.zeros(shape, dtype=torch.int64, device=A.device)
    elif (trace.dtype != torch.int64 or tuple(trace.shape) != shape or not trace.is_contiguous()
          or trace.device != A.device):
        raise ValueError("trace must be a contiguous int64 [%d, %d] tensor on A's device" % shape)
    st = lib.gg_trace_grouped_gemm_bf16(A.data_ptr(), B.data_ptr(), offsets.data_ptr(),
                                        out.data_ptr(), E, K, N, M_cap, int(bm), trace.data_ptr(),
                                        int(max_tiles), _stream_handle(A.device, stream))
    if st != 0:
        raise GroupedGemmError("gg_trace_grouped_gemm_bf16: status %d (%s)"
                               % (st, lib.gg_status_string(st).decode()))
    khz = ctypes.c_int32(0)
    st = lib.gg_trace_clock_khz(ctypes.byref(khz))
    if st != 0:
        raise GroupedGemmError("gg_trace_clock_khz: status %d" % st)
    return out, trace, int(khz.value)
