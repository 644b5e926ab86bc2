"""Python binding of libmkp (run-time polymerized dense GEMM for MI355X).

Argument marshalling only: every step of the GEMM (plan lookup, the
polymerizer, every kernel) runs inside libmkp.so.  PyTorch is used only to
hand over device pointers and the current HIP stream.  If the library has not
been built this module raises on import: there is no fallback path.

Names follow the C-ABI in include/mkp.h: mkp_gemm(M,N,K,A,lda,B,ldb,C,ldc,
stream) and mkp_gemm_batched(...).
"""
from __future__ import annotations

import ctypes
import json
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmkp.so")

MKP_OK = 0
MKP_ERR_INVALID_ARG = -1
MKP_ERR_UNSUPPORTED = -2
MKP_ERR_OOM = -3
MKP_ERR_HIP = -4
MKP_ERR_BUFFER = -5
MKP_PLAN_EXHAUSTIVE = 1
MKP_PLAN_B_NK = 8
MKP_B_KN = 0
MKP_B_NK = 1
MKP_ACT_NONE = 0
MKP_ACT_RELU = 1
MKP_ACT_GELU = 2
MKP_ACT_GELU_TANH = 3
MKP_ACT_SILU = 4
ACTIVATIONS = {None: MKP_ACT_NONE, "none": MKP_ACT_NONE, "relu": MKP_ACT_RELU, "gelu": MKP_ACT_GELU,
               "gelu_tanh": MKP_ACT_GELU_TANH, "silu": MKP_ACT_SILU}


class MkpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mkp error {code}: {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python dynamic_shape_gemm_amd/build.py`")

# One HIP runtime per process.  The PyTorch wheel carries its own copy of the
# HIP and HSA runtimes under the same soname as the system's; whichever is
# loaded first is the one libmkp binds to.  If libmkp came first, torch would
# load a second runtime beside it and libmkp's would find no device.  So
# torch, when installed, is loaded before the library.
try:
    import torch  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(LIB_PATH)
_i64, _p, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
_lib.mkp_gemm.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.mkp_gemm.restype = _int
_lib.mkp_gemm_batched.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p]
_lib.mkp_gemm_batched.restype = _int
_lib.mkp_gemm_batched_noalloc.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p]
_lib.mkp_gemm_batched_noalloc.restype = _int
_lib.mkp_noalloc_scratch_bytes.argtypes = []
_lib.mkp_noalloc_scratch_bytes.restype = ctypes.c_size_t
_lib.mkp_gemm_bt.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.mkp_gemm_bt.restype = _int
_lib.mkp_gemm_batched_bt.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _p]
_lib.mkp_gemm_batched_bt.restype = _int
_lib.mkp_gemm_ex.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _int, _p, _i64, _i64,
                             ctypes.c_float, ctypes.c_float, _p, _int, _p]
_lib.mkp_gemm_ex.restype = _int
_lib.mkp_conv2d.argtypes = [_i64] * 13 + [_p, _p, _p, _p, _int, _p]
_lib.mkp_conv2d.restype = _int
_grp_args = [_i64, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p, _p]
_lib.mkp_gemm_grouped.argtypes = _grp_args
_lib.mkp_gemm_grouped.restype = _int
_lib.mkp_gemm_grouped_bt.argtypes = _grp_args
_lib.mkp_gemm_grouped_bt.restype = _int
_lib.mkp_plan_describe_grouped.argtypes = [_i64, _i64, _i64, _p, _int, ctypes.c_char_p, ctypes.c_size_t]
_lib.mkp_plan_describe_grouped.restype = _int
_lib.mkp_plan_describe.argtypes = [_i64, _i64, _i64, _i64, _int, ctypes.c_char_p, ctypes.c_size_t]
_lib.mkp_plan_describe.restype = _int
_lib.mkp_plan_with_table.argtypes = [ctypes.c_char_p, _int, _i64, _i64, _i64, _i64, ctypes.c_char_p, ctypes.c_size_t]
_lib.mkp_plan_with_table.restype = _int
_lib.mkp_load_calibration.argtypes = [ctypes.c_char_p]
_lib.mkp_load_calibration.restype = _int
_lib.mkp_calibrate.argtypes = [ctypes.c_char_p, _int]
_lib.mkp_calibrate.restype = _int
_lib.mkp_set_option.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
_lib.mkp_set_option.restype = _int
_lib.mkp_kernel_count.argtypes = []
_lib.mkp_kernel_count.restype = _int
_lib.mkp_kernel_name.argtypes = [_int]
_lib.mkp_kernel_name.restype = ctypes.c_char_p
_lib.mkp_cache_clear.argtypes = []
_lib.mkp_cache_clear.restype = None
_lib.mkp_stats.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
_lib.mkp_stats.restype = _int
_lib.mkp_trace_dump.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
_lib.mkp_trace_dump.restype = _int
_lib.mkp_last_error.argtypes = []
_lib.mkp_last_error.restype = ctypes.c_char_p

# The GEMM entry points through the CPython marshalling module built beside
# the library (a ctypes call spends ~1.5 us converting 10-14 arguments, as
# long as the smallest GEMMs take on the GPU); ctypes where it is absent.
try:
    from . import _mkpfast as _fast
except ImportError:
    _fast = None
_f_gemm = _fast.gemm if _fast else _lib.mkp_gemm
_f_gemm_bt = _fast.gemm_bt if _fast else _lib.mkp_gemm_bt
_f_gemm_batched = _fast.gemm_batched if _fast else _lib.mkp_gemm_batched
_f_gemm_batched_bt = _fast.gemm_batched_bt if _fast else _lib.mkp_gemm_batched_bt

EXPORTED = ["mkp_gemm", "mkp_gemm_batched", "mkp_gemm_batched_noalloc", "mkp_noalloc_scratch_bytes", "mkp_gemm_bt", "mkp_gemm_batched_bt", "mkp_gemm_ex", "mkp_conv2d", "mkp_gemm_grouped",
            "mkp_gemm_grouped_bt", "mkp_plan_describe", "mkp_plan_describe_grouped", "mkp_plan_with_table",
            "mkp_load_calibration",
            "mkp_calibrate", "mkp_set_option", "mkp_kernel_count", "mkp_kernel_name", "mkp_cache_clear",
            "mkp_stats", "mkp_trace_dump", "mkp_last_error"]


def last_error() -> str:
    return (_lib.mkp_last_error() or b"").decode()


def _check(rc: int) -> int:
    if rc != MKP_OK:
        raise MkpError(rc, last_error())
    return rc


def _addr(x) -> int:
    """Device address of a torch tensor, or an int address as given."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def mkp_gemm(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    """C[MxN] := A[MxK] . B[KxN] (bf16 in, fp32 out), enqueued on `stream`
    (default: torch's current stream).  Raises MkpError on a bad argument."""
    return _check(_f_gemm(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, _stream(stream)))


def mkp_gemm_batched(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, stream=None) -> int:
    return _check(_f_gemm_batched(batch, M, N, K, _addr(A), lda, strideA, _addr(B), ldb, strideB, _addr(C),
                                  ldc, strideC, _stream(stream)))


def mkp_gemm_batched_noalloc(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, stream=None) -> int:
    """mkp_gemm_batched without any device allocation: its scratch is the
    library's fixed per-GPU array (calls that overlap on one GPU race)."""
    return _check(_lib.mkp_gemm_batched_noalloc(batch, M, N, K, _addr(A), lda, strideA, _addr(B), ldb, strideB,
                                                _addr(C), ldc, strideC, _stream(stream)))


def mkp_noalloc_scratch_bytes() -> int:
    return int(_lib.mkp_noalloc_scratch_bytes())


def mkp_gemm_raw(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    """As mkp_gemm but returns the status code instead of raising."""
    return _f_gemm(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, stream or 0)


def mkp_gemm_batched_raw(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream) -> int:
    return _f_gemm_batched(batch, M, N, K, _addr(A), lda, sA, _addr(B), ldb, sB, _addr(C), ldc, sC, stream or 0)


def mkp_gemm_bt(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    """C[MxN] := A[MxK] . B^T with B given as N x K (ldb >= K)."""
    return _check(_f_gemm_bt(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, _stream(stream)))


def mkp_gemm_batched_bt(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, stream=None) -> int:
    return _check(_f_gemm_batched_bt(batch, M, N, K, _addr(A), lda, strideA, _addr(B), ldb, strideB,
                                     _addr(C), ldc, strideC, _stream(stream)))


def mkp_gemm_bt_raw(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return _f_gemm_bt(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, stream or 0)


def mkp_gemm_batched_bt_raw(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream) -> int:
    return _f_gemm_batched_bt(batch, M, N, K, _addr(A), lda, sA, _addr(B), ldb, sB, _addr(C), ldc, sC,
                              stream or 0)


def mkp_gemm_ex(batch, M, N, K, A, lda, strideA, B, ldb, strideB, b_layout, C, ldc, strideC,
                alpha=1.0, beta=0.0, bias=None, act=MKP_ACT_NONE, stream=None) -> int:
    """C_b := act(alpha * A_b . op(B_b) + beta * C_b + bias) with op(B) = B
    (b_layout MKP_B_KN) or B^T (MKP_B_NK); act an MKP_ACT_* code or name."""
    return _check(mkp_gemm_ex_raw(batch, M, N, K, A, lda, strideA, B, ldb, strideB, b_layout, C, ldc, strideC,
                                  alpha, beta, bias, act, _stream(stream)))


def mkp_gemm_ex_raw(batch, M, N, K, A, lda, strideA, B, ldb, strideB, b_layout, C, ldc, strideC,
                    alpha, beta, bias, act, stream) -> int:
    if not isinstance(act, int):
        act = ACTIVATIONS[act]
    return _lib.mkp_gemm_ex(batch, M, N, K, _addr(A), lda, strideA, _addr(B), ldb, strideB, b_layout, _addr(C), ldc,
                            strideC, alpha, beta, _addr(bias), act, stream or 0)


def mkp_conv2d_raw(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y, bias=None,
                   act=MKP_ACT_NONE, stream=0) -> int:
    if not isinstance(act, int):
        act = ACTIVATIONS[act]
    return _lib.mkp_conv2d(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, _addr(x), _addr(w),
                           _addr(y), _addr(bias), act, stream or 0)


def mkp_conv2d(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y, bias=None,
               act=MKP_ACT_NONE, stream=None) -> int:
    """y (N,P,Q,K) fp32 := act(conv2d(x (N,H,W,C) bf16, w (K,R,S,C) bf16) + bias)."""
    return _check(mkp_conv2d_raw(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, x, w, y,
                                 bias, act, _stream(stream)))


def conv_out_size(H, R, stride, pad, dil):
    return (H + 2 * pad - dil * (R - 1) - 1) // stride + 1


def _i64_array(values):
    return (ctypes.c_int64 * max(len(values), 1))(*[int(v) for v in values])


def _ptr_array(values):
    return (ctypes.c_void_p * max(len(values), 1))(*[_addr(v) for v in values])


def _grouped_call(fn, M, K, A, lda, N, B, ldb, C, ldc, stream):
    g = len(N)
    if not (len(B) == len(ldb) == len(C) == len(ldc) == g):
        raise ValueError("N, B, ldb, C and ldc must have one entry per group")
    return fn(g, M, K, _addr(A), lda, ctypes.cast(_i64_array(N), _p), ctypes.cast(_ptr_array(B), _p),
              ctypes.cast(_i64_array(ldb), _p), ctypes.cast(_ptr_array(C), _p), ctypes.cast(_i64_array(ldc), _p),
              stream)


def mkp_gemm_grouped(M, K, A, lda, N, B, ldb, C, ldc, stream=None) -> int:
    """C[g][M x N[g]] := A[M x K] . B[g] (B[g] K x N[g]) for every group, in
    one launch.  N, B, ldb, C, ldc are sequences with one entry per group."""
    return _check(_grouped_call(_lib.mkp_gemm_grouped, M, K, A, lda, N, B, ldb, C, ldc, _stream(stream)))


def mkp_gemm_grouped_bt(M, K, A, lda, N, B, ldb, C, ldc, stream=None) -> int:
    """As mkp_gemm_grouped with each B[g] given as N[g] x K (ldb[g] >= K)."""
    return _check(_grouped_call(_lib.mkp_gemm_grouped_bt, M, K, A, lda, N, B, ldb, C, ldc, _stream(stream)))


def mkp_gemm_grouped_raw(M, K, A, lda, N, B, ldb, C, ldc, stream, bt=False) -> int:
    fn = _lib.mkp_gemm_grouped_bt if bt else _lib.mkp_gemm_grouped
    return _grouped_call(fn, M, K, A, lda, N, B, ldb, C, ldc, stream or 0)


def mkp_plan_describe_grouped(M, K, N, bt=False) -> dict:
    return json.loads(_text_call(_lib.mkp_plan_describe_grouped, len(N), M, K,
                                 ctypes.cast(_i64_array(N), _p), MKP_PLAN_B_NK if bt else 0))


def _text_call(fn, *args, size=1 << 16):
    buf = ctypes.create_string_buffer(size)
    _check(fn(*args, buf, size))
    return buf.value.decode()


def mkp_plan_describe(batch, M, N, K, align_flags=7, bt=False) -> dict:
    return json.loads(_text_call(_lib.mkp_plan_describe, batch, M, N, K,
                                 align_flags | (MKP_PLAN_B_NK if bt else 0)))


def mkp_plan_with_table(table_text: str, batch, M, N, K, exhaustive=False, bt=False) -> dict:
    flags = (MKP_PLAN_EXHAUSTIVE if exhaustive else 0) | (MKP_PLAN_B_NK if bt else 0)
    return json.loads(_text_call(_lib.mkp_plan_with_table, table_text.encode(), flags, batch, M, N, K))


def mkp_load_calibration(path=None) -> int:
    return _check(_lib.mkp_load_calibration(path.encode() if path else None))


def mkp_calibrate(path: str, max_points: int = 0) -> int:
    return _check(_lib.mkp_calibrate(path.encode(), max_points))


def mkp_set_option(key: str, value) -> int:
    return _check(_lib.mkp_set_option(key.encode(), str(value).encode()))


def mkp_kernel_names() -> list:
    return [_lib.mkp_kernel_name(i).decode() for i in range(_lib.mkp_kernel_count())]


def mkp_cache_clear() -> None:
    _lib.mkp_cache_clear()


def mkp_stats() -> dict:
    return json.loads(_text_call(_lib.mkp_stats))


def mkp_trace_dump() -> list:
    return json.loads(_text_call(_lib.mkp_trace_dump, size=1 << 24))


def gemm(a, b, out=None, stream=None):
    """torch convenience: a (M,K) bf16, b (K,N) bf16 on the GPU, any strides
    with unit column stride; returns (or fills) out (M,N) fp32."""
    import torch
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("a and b must be bfloat16")
    if a.stride(1) != 1 or b.stride(1) != 1:
        raise ValueError("rows must be contiguous (unit column stride)")
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    mkp_gemm(M, N, K, a, max(a.stride(0), 1), b, max(b.stride(0), 1), out, max(out.stride(0), 1), stream)
    return out


def gemm_batched(a, b, out=None, stream=None):
    """torch convenience: a (batch,M,K), b (batch,K,N) bf16 -> out (batch,M,N) fp32."""
    import torch
    batch, M, K = a.shape
    N = b.shape[2]
    if out is None:
        out = torch.empty((batch, M, N), dtype=torch.float32, device=a.device)
    mkp_gemm_batched(batch, M, N, K, a, max(a.stride(1), 1), a.stride(0), b, max(b.stride(1), 1), b.stride(0),
                     out, max(out.stride(1), 1), out.stride(0), stream)
    return out


def gemm_bt(a, w, out=None, stream=None):
    """torch convenience: a (M,K) bf16 and w (N,K) bf16 (a linear layer's
    weight) on the GPU, unit column strides; returns (or fills) out = a . w^T
    (M,N) fp32."""
    import torch
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("a and w must be bfloat16")
    if a.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("rows must be contiguous (unit column stride)")
    M, K = a.shape
    N, K2 = w.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    mkp_gemm_bt(M, N, K, a, max(a.stride(0), 1), w, max(w.stride(0), 1), out, max(out.stride(0), 1), stream)
    return out


def gemm_grouped(a, ws, outs=None, stream=None, bt=False):
    """torch convenience: one A (M,K) bf16 against several weights in one
    launch.  ws: list of (K,N_g) bf16 tensors, or (N_g,K) with bt=True.
    Returns (or fills) the list of (M,N_g) fp32 outputs."""
    import torch
    if a.dtype != torch.bfloat16 or any(w.dtype != torch.bfloat16 for w in ws):
        raise TypeError("a and the weights must be bfloat16")
    if a.stride(1) != 1 or any(w.stride(1) != 1 for w in ws):
        raise ValueError("rows must be contiguous (unit column stride)")
    M, K = a.shape
    Ns = [w.shape[0] if bt else w.shape[1] for w in ws]
    if any((w.shape[1] if bt else w.shape[0]) != K for w in ws):
        raise ValueError("inner dimensions differ")
    if outs is None:
        outs = [torch.empty((M, n), dtype=torch.float32, device=a.device) for n in Ns]
    if any(o.stride(1) != 1 for o in outs):
        raise ValueError("out rows must be contiguous")
    fn = mkp_gemm_grouped_bt if bt else mkp_gemm_grouped
    fn(M, K, a, max(a.stride(0), 1), Ns, ws, [max(w.stride(0), 1) for w in ws], outs,
       [max(o.stride(0), 1) for o in outs], stream)
    return outs


def linear(a, w, bias=None, act=None, out=None, beta=0.0, stream=None):
    """torch convenience for a linear layer: out = act(a . w^T + bias (+ beta
    * out)), a (M,K) bf16, w (N,K) bf16 (the layer's weight), bias (N,) fp32
    or None, act None/"relu"/"gelu"/"gelu_tanh"/"silu"; all in one launch
    sequence of the library (the epilogue runs inside the GEMM)."""
    import torch
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("a and w must be bfloat16")
    if bias is not None and (bias.dtype != torch.float32 or bias.stride(0) != 1):
        raise TypeError("bias must be a contiguous float32 vector")
    if a.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("rows must be contiguous (unit column stride)")
    M, K = a.shape
    N, K2 = w.shape
    if K2 != K or (bias is not None and bias.shape[0] != N):
        raise ValueError("shapes differ")
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs out")
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    mkp_gemm_ex(1, M, N, K, a, max(a.stride(0), 1), 0, w, max(w.stride(0), 1), 0, MKP_B_NK, out,
                max(out.stride(0), 1), 0, 1.0, beta, bias, act, stream)
    return out


def conv2d(x, w, bias=None, act=None, stride=1, padding=0, dilation=1, out=None, stream=None):
    """torch convenience: x (N,H,W,C) bf16 NHWC, w (K,R,S,C) bf16, contiguous;
    returns (or fills) y (N,P,Q,K) fp32 = act(conv2d(x, w) + bias)."""
    import torch
    sh, sw = (stride, stride) if isinstance(stride, int) else stride
    ph, pw = (padding, padding) if isinstance(padding, int) else padding
    dh, dw = (dilation, dilation) if isinstance(dilation, int) else dilation
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("x and w must be bfloat16")
    if not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("x and w must be contiguous (NHWC and KRSC)")
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    if C2 != C:
        raise ValueError("channel counts differ")
    P, Q = conv_out_size(H, R, sh, ph, dh), conv_out_size(W, S, sw, pw, dw)
    if out is None:
        out = torch.empty((N, P, Q, K), dtype=torch.float32, device=x.device)
    mkp_conv2d(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, x, w, out, bias, act, stream)
    return out
