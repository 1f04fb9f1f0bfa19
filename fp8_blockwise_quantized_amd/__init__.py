"""Python binding of libfp8bq (FP8 blockwise-quantized linear layer for MI355X / gfx950).

Argument marshalling only: every function below passes torch tensors' device pointers, sizes,
leading dimensions and the current HIP stream to the C-ABI entry point of the same name declared in
``include/fp8bq.h``; all computation happens in the library's HIP kernels.  PyTorch provides device
memory and streams.  If the library is not built, importing the binding's functions raises.

Raw entry points (same names and argument order as the C ABI, tensors in place of pointers):

    fp8bq_quantize_act_1x128(x, fmt, q, s)
    fp8bq_quantize_act_128x1(x, fmt, qt, st)
    fp8bq_quantize_act_dual(x, fmt_rows, q, s, fmt_cols, qt, st)
    fp8bq_quantize_weight_128x128(w, fmt, q, s)
    fp8bq_quantize_weight_dual(w, fmt, q, s, qt)
    fp8bq_quantize_weights_dual(jobs, fmt)    jobs: up to 16 (w, q, s, qt) tuples, one launch
    fp8bq_hyperball_step_batch(jobs, lr, wd, eps, ws)  jobs: up to 32 (w, g, radius, norms) tuples, two launches
    fp8bq_gemm_fprop(qx, sx, fx, qw, sw, fw, y, ws=None)
    fp8bq_gemm_dgrad(qdy, sdy, fdy, qw, sw, fw, dx, ws=None)
    fp8bq_gemm_dgrad_wt(qdy, sdy, fdy, qwt, sw, fw, dx, ws=None)
    fp8bq_gemm_wgrad(qdyt, sdyt, fdy, qxt, sxt, fx, dw, ws=None)
    fp8bq_gemm_workspace_size(op, M, N, K)
    fp8bq_gemm_plan(op, M, N, K) -> (tile_m, tile_n, split_k)
    fp8bq_quantize_tensor_delayed(x, fmt, amax, beta, q, qt, s, ws)
    fp8bq_quantize_tensor_delayed_noalloc(x, fmt, amax, beta, q, qt, s)   (the library's own scratch)

Allocating helpers (outputs created with torch on the input's device):

    quantize_act_1x128(x, fmt) -> (q [R, C] uint8, s [C/128, R] float32)
    quantize_act_128x1(x, fmt) -> (qt [C, R] uint8, st [R/128, C] float32)
    quantize_act_dual(x, fmt_rows, fmt_cols) -> (q, s, qt, st) of the two above, one pass over x
    quantize_weight_128x128(w, fmt) -> (q [N, K] uint8, s [N/128, K/128] float32)
    quantize_weight_dual(w, fmt) -> (q, s, qt [K, N]): the above plus the transposed codes
    quantize_weights_dual(ws, fmt) -> [(q, s, qt), ...]: quantize_weight_dual of every weight in ws,
        in one launch per 16 weights
    gemm_fprop(qx, sx, qw, sw, fx=E4M3, fw=E4M3, out_dtype=bf16) -> y [M, N]
    gemm_dgrad(qdy, sdy, qw, sw, fdy=E4M3, fw=E4M3, out_dtype=bf16) -> dx [M, K]
    gemm_dgrad_wt(qdy, sdy, qwt, sw, fdy=E4M3, fw=E4M3, out_dtype=bf16) -> dx [M, K] (qwt = W^T codes)
    gemm_wgrad(qdyt, sdyt, qxt, sxt, fdy=E4M3, fx=E4M3, out_dtype=bf16, accumulate=False) -> dw [N, K]
    quantize_tensor_delayed(x, amax, beta=0.99, fmt=E4M3, transpose=False) -> (q, s, qt or None):
        per-tensor delayed scaling (running amax updated in place, one scale per tensor)
    gemm_tensor(qa, sa, qb, sb, fa=E4M3, fb=E4M3, out_dtype=bf16) -> y [M, N] (per-tensor scales)
    hyperball_step(w, g, lr=1e-4, weight_decay=0.1, eps=1e-8, radius=0.0) -> norms:
        in-place normalized update of an FP32 weight (and projection onto `radius` if > 0)
        (accumulate=True: out, an FP32 main-grad buffer, receives out + dW)
"""

import ctypes
import os

import torch

E4M3 = 0
E5M2 = 1
IN_BF16 = 0
IN_F32 = 1
OUT_BF16 = 0
OUT_F32 = 1
OUT_F32_ACCUM = 2  # wgrad only: the FP32 output receives out + result
OP_FPROP = 0
OP_DGRAD = 1
OP_WGRAD = 2
OP_DGRAD_WT = 3
OP_TENSOR = 4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libfp8bq.so")

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_vp = ctypes.c_void_p
_c_sz = ctypes.c_size_t


class WeightJob(ctypes.Structure):
    """fp8bq_weight_job of the C ABI: one weight of fp8bq_quantize_weights_dual."""
    _fields_ = [("w", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("ldw", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("ldq", ctypes.c_int64), ("s", ctypes.c_void_p), ("lds", ctypes.c_int64),
                ("qt", ctypes.c_void_p), ("ldqt", ctypes.c_int64)]


MAX_WEIGHT_JOBS = 16


class HyperballJob(ctypes.Structure):
    """fp8bq_hyperball_job of the C ABI: one matrix of fp8bq_hyperball_step_batch."""
    _fields_ = [("w", ctypes.c_void_p), ("ldw", ctypes.c_int64), ("g", ctypes.c_void_p), ("ldg", ctypes.c_int64),
                ("R", ctypes.c_int64), ("C", ctypes.c_int64), ("radius", ctypes.c_double), ("norms", ctypes.c_void_p)]


MAX_HYPERBALL_JOBS = 32

_SIGS = {
    "fp8bq_quantize_act_1x128": [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp],
    "fp8bq_quantize_act_128x1": [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp],
    "fp8bq_quantize_act_dual": [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64, _c_int,
                                _c_vp, _c_i64, _c_vp, _c_i64, _c_vp],
    "fp8bq_quantize_weight_dual": [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp,
                                   _c_i64, _c_vp],
    "fp8bq_quantize_weights_dual": [ctypes.POINTER(WeightJob), _c_int, _c_int, _c_int, _c_vp],
    "fp8bq_quantize_weight_128x128": [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64,
                                      _c_vp],
    "fp8bq_gemm_fprop": [_c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64,
                         _c_int, _c_vp, _c_int, _c_i64, _c_vp, _c_sz, _c_vp],
    "fp8bq_gemm_dgrad": [_c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64,
                         _c_int, _c_vp, _c_int, _c_i64, _c_vp, _c_sz, _c_vp],
    "fp8bq_gemm_dgrad_wt": [_c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_int, _c_vp, _c_i64, _c_vp,
                            _c_i64, _c_int, _c_vp, _c_int, _c_i64, _c_vp, _c_sz, _c_vp],
    "fp8bq_gemm_wgrad": [_c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_i64, _c_int, _c_vp, _c_i64, _c_vp, _c_i64,
                         _c_int, _c_vp, _c_int, _c_i64, _c_vp, _c_sz, _c_vp],
    "fp8bq_gemm_tensor": [_c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_int, _c_vp, _c_i64, _c_vp, _c_int, _c_vp,
                          _c_int, _c_i64, _c_vp, _c_sz, _c_vp],
    "fp8bq_quantize_tensor_workspace_size": [_c_i64, _c_i64],
    "fp8bq_quantize_tensor_delayed": [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, ctypes.c_double, _c_vp,
                                      _c_i64, _c_vp, _c_i64, _c_vp, _c_vp, _c_sz, _c_vp],
    "fp8bq_quantize_tensor_delayed_noalloc": [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, ctypes.c_double,
                                              _c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_vp],
    "fp8bq_hyperball_workspace_size": [_c_i64, _c_i64],
    "fp8bq_hyperball_step": [_c_vp, _c_i64, _c_vp, _c_int, _c_i64, _c_i64, _c_i64, ctypes.c_double, ctypes.c_double,
                             ctypes.c_double, ctypes.c_double, _c_vp, _c_vp, _c_sz, _c_vp],
    "fp8bq_gemm_workspace_size": [_c_int, _c_i64, _c_i64, _c_i64],
    "fp8bq_gemm_plan": [_c_int, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp],
    "fp8bq_stream_copy": [_c_vp, _c_vp, _c_sz, _c_vp],
    "fp8bq_hyperball_batch_workspace_size": [_c_int],
    "fp8bq_hyperball_step_batch": [ctypes.POINTER(HyperballJob), _c_int, _c_int, ctypes.c_double, ctypes.c_double,
                                   ctypes.c_double, _c_vp, _c_sz, _c_vp],
    "fp8bq_status_string": [_c_int],
    "fp8bq_version": [],
}
_RESTYPES = {"fp8bq_gemm_workspace_size": _c_sz, "fp8bq_quantize_tensor_workspace_size": _c_sz,
             "fp8bq_hyperball_workspace_size": _c_sz,
             "fp8bq_hyperball_batch_workspace_size": _c_sz,
             "fp8bq_status_string": ctypes.c_char_p}

_lib = None


class Fp8bqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def lib():
    """The loaded ctypes library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libfp8bq.so is not built ({LIB_PATH}); run `python -m fp8_blockwise_quantized_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, _c_int)
        _lib = handle
    return _lib


def status_string(status):
    return lib().fp8bq_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise Fp8bqError(status, where)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ld(t):
    if t.dim() == 2 and t.numel() == 0:
        return t.size(1)  # an empty matrix has no meaningful strides; the call does nothing with it
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


def _in_type(t):
    if t.dtype == torch.bfloat16:
        return IN_BF16
    if t.dtype == torch.float32:
        return IN_F32
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _out_type(t):
    if t.dtype == torch.bfloat16:
        return OUT_BF16
    if t.dtype == torch.float32:
        return OUT_F32
    raise TypeError(f"unsupported output dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_HI = (torch.bfloat16, torch.float32)


def _expect_all(checks, ws=None):
    """Refuse, before any launch, tensors the C call would misread: the C ABI sees only pointers and
    leading dimensions, so it cannot check a buffer's extent, element type or device.  checks:
    (tensor or None, name, shape, dtypes); every tensor's dtype and shape first, then that all (and
    the workspace ws, if any) are on the first tensor's device, a CUDA (HIP) device."""
    for t, name, shape, dtypes in checks:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.dtype not in dtypes:
            raise TypeError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
        if t.shape != shape:
            raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    device = checks[0][0].device
    if device.type != "cuda":
        raise ValueError(f"{checks[0][1]} must be on a CUDA (HIP) device, not {device}")
    for t, name, _, _ in checks[1:]:
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the call's tensors on {device}")
    if ws is not None:
        if not isinstance(ws, torch.Tensor):
            raise TypeError("ws must be a torch tensor or None")
        if not ws.is_contiguous():
            raise ValueError("ws must be contiguous")
        if ws.device != device:
            raise ValueError(f"ws is on {ws.device}, the call's tensors on {device}")


# ---------------------------------------------------------------------------------------------
# raw entry points
# ---------------------------------------------------------------------------------------------

_MARSHAL = {}


def _entry(marshal):
    """Make an entry point from a function that validates its tensors and returns the C call's
    argument tuple: calling the entry point marshals and launches; prepare() keeps the marshalled
    arguments for repeated launches."""
    name = marshal.__name__
    _MARSHAL[name] = marshal

    def call(*args, **kwargs):
        _check(getattr(lib(), name)(*marshal(*args, **kwargs)), name)

    call.__name__ = name
    call.__qualname__ = name
    call.__doc__ = marshal.__doc__
    return call


def prepare(fn, *args, **kwargs):
    """Validate and marshal the arguments of raw entry point `fn` once and return a function that
    launches `fn` with them (on the stream current at preparation): the repeated calls of a training
    or serving loop then cost one C call each.  The tensors must stay alive and keep their storage."""
    name = fn.__name__
    cargs = _MARSHAL[name](*args, **kwargs)
    cfn = getattr(lib(), name)

    def launch():
        st = cfn(*cargs)
        if st != 0:
            raise Fp8bqError(st, name)

    return launch


@_entry
def fp8bq_quantize_act_1x128(x, fmt, q, s):
    R, C = x.shape
    _expect_all([(x, "x", (R, C), _HI), (q, "q", (R, C), _U8), (s, "s", (C // 128, R), _F32)])
    return (_ptr(x), _in_type(x), R, C, _ld(x), fmt, _ptr(q), _ld(q), _ptr(s), _ld(s),
            _stream(x))


@_entry
def fp8bq_quantize_act_128x1(x, fmt, qt, st):
    R, C = x.shape
    _expect_all([(x, "x", (R, C), _HI), (qt, "qt", (C, R), _U8), (st, "st", (R // 128, C), _F32)])
    return (_ptr(x), _in_type(x), R, C, _ld(x), fmt, _ptr(qt), _ld(qt), _ptr(st),
            _ld(st), _stream(x))


@_entry
def fp8bq_quantize_act_dual(x, fmt_rows, q, s, fmt_cols, qt, st):
    R, C = x.shape
    _expect_all([(x, "x", (R, C), _HI), (q, "q", (R, C), _U8), (s, "s", (C // 128, R), _F32),
                 (qt, "qt", (C, R), _U8), (st, "st", (R // 128, C), _F32)])
    return (_ptr(x), _in_type(x), R, C, _ld(x), fmt_rows, _ptr(q), _ld(q), _ptr(s),
            _ld(s), fmt_cols, _ptr(qt), _ld(qt), _ptr(st), _ld(st), _stream(x))


@_entry
def fp8bq_quantize_weight_dual(w, fmt, q, s, qt):
    N, K = w.shape
    _expect_all([(w, "w", (N, K), _HI), (q, "q", (N, K), _U8),
                 (s, "s", (N // 128, K // 128), _F32), (qt, "qt", (K, N), _U8)])
    return (_ptr(w), _in_type(w), N, K, _ld(w), fmt, _ptr(q), _ld(q), _ptr(s), _ld(s),
            _ptr(qt), _ld(qt), _stream(w))


@_entry
def fp8bq_quantize_weights_dual(jobs, fmt):
    """jobs: (w, q, s, qt) per weight, as fp8bq_quantize_weight_dual takes them; every w of one dtype.
    One launch on the current stream of the first weight's device."""
    jobs = list(jobs)
    arr = (WeightJob * max(len(jobs), 1))()
    wt = _in_type(jobs[0][0]) if jobs else IN_BF16
    if any(_in_type(job[0]) != wt for job in jobs):
        raise TypeError("all weights of one fp8bq_quantize_weights_dual call must share one dtype")
    for i, (w, q, s, qt) in enumerate(jobs):
        N, K = w.shape
        _expect_all([(jobs[0][0], "jobs[0].w", jobs[0][0].shape, _HI), (w, f"jobs[{i}].w", (N, K), _HI),
                     (q, f"jobs[{i}].q", (N, K), _U8), (s, f"jobs[{i}].s", (N // 128, K // 128), _F32),
                     (qt, f"jobs[{i}].qt", (K, N), _U8)])
        arr[i] = WeightJob(w.data_ptr(), N, K, _ld(w), q.data_ptr(), _ld(q), s.data_ptr(), _ld(s), qt.data_ptr(),
                           _ld(qt))
    stream = _stream(jobs[0][0]) if jobs else ctypes.c_void_p(0)
    return (arr, len(jobs), wt, fmt, stream)


@_entry
def fp8bq_quantize_weight_128x128(w, fmt, q, s):
    N, K = w.shape
    _expect_all([(w, "w", (N, K), _HI), (q, "q", (N, K), _U8),
                 (s, "s", (N // 128, K // 128), _F32)])
    return (_ptr(w), _in_type(w), N, K, _ld(w), fmt, _ptr(q), _ld(q), _ptr(s),
            _ld(s), _stream(w))


def fp8bq_gemm_workspace_size(op, M, N, K):
    return int(lib().fp8bq_gemm_workspace_size(int(op), int(M), int(N), int(K)))


def fp8bq_gemm_plan(op, M, N, K):
    tm, tn, sk = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = lib().fp8bq_gemm_plan(int(op), int(M), int(N), int(K), ctypes.cast(ctypes.byref(tm), _c_vp),
                               ctypes.cast(ctypes.byref(tn), _c_vp), ctypes.cast(ctypes.byref(sk), _c_vp))
    _check(st, "fp8bq_gemm_plan")
    return tm.value, tn.value, sk.value


def _ws_args(ws):
    if ws is None:
        return ctypes.c_void_p(0), 0
    return _ptr(ws), ws.numel() * ws.element_size()


@_entry
def fp8bq_gemm_fprop(qx, sx, fx, qw, sw, fw, y, ws=None):
    M, K = qx.shape
    N = qw.shape[0]
    _expect_all([(qx, "qx", (M, K), _U8), (sx, "sx", (K // 128, M), _F32), (qw, "qw", (N, K), _U8),
                 (sw, "sw", (N // 128, K // 128), _F32), (y, "y", (M, N), _HI)], ws)
    wsp, wsb = _ws_args(ws)
    return (M, N, K, _ptr(qx), _ld(qx), _ptr(sx), _ld(sx), fx, _ptr(qw), _ld(qw), _ptr(sw),
            _ld(sw), fw, _ptr(y), _out_type(y), _ld(y), wsp, wsb, _stream(y))


@_entry
def fp8bq_gemm_dgrad(qdy, sdy, fdy, qw, sw, fw, dx, ws=None):
    M, N = qdy.shape
    K = qw.shape[1]
    _expect_all([(qdy, "qdy", (M, N), _U8), (sdy, "sdy", (N // 128, M), _F32), (qw, "qw", (N, K), _U8),
                 (sw, "sw", (N // 128, K // 128), _F32), (dx, "dx", (M, K), _HI)], ws)
    wsp, wsb = _ws_args(ws)
    return (M, N, K, _ptr(qdy), _ld(qdy), _ptr(sdy), _ld(sdy), fdy, _ptr(qw), _ld(qw),
            _ptr(sw), _ld(sw), fw, _ptr(dx), _out_type(dx), _ld(dx), wsp, wsb, _stream(dx))


@_entry
def fp8bq_gemm_dgrad_wt(qdy, sdy, fdy, qwt, sw, fw, dx, ws=None):
    M, N = qdy.shape
    K = qwt.shape[0]
    _expect_all([(qdy, "qdy", (M, N), _U8), (sdy, "sdy", (N // 128, M), _F32), (qwt, "qwt", (K, N), _U8),
                 (sw, "sw", (N // 128, K // 128), _F32), (dx, "dx", (M, K), _HI)], ws)
    wsp, wsb = _ws_args(ws)
    return (M, N, K, _ptr(qdy), _ld(qdy), _ptr(sdy), _ld(sdy), fdy, _ptr(qwt), _ld(qwt),
            _ptr(sw), _ld(sw), fw, _ptr(dx), _out_type(dx), _ld(dx), wsp, wsb, _stream(dx))


@_entry
def fp8bq_gemm_wgrad(qdyt, sdyt, fdy, qxt, sxt, fx, dw, ws=None, accumulate=False):
    N, M = qdyt.shape
    K = qxt.shape[0]
    _expect_all([(qdyt, "qdyt", (N, M), _U8), (sdyt, "sdyt", (M // 128, N), _F32), (qxt, "qxt", (K, M), _U8),
                 (sxt, "sxt", (M // 128, K), _F32), (dw, "dw", (N, K), _F32 if accumulate else _HI)], ws)
    wsp, wsb = _ws_args(ws)
    ot = OUT_F32_ACCUM if accumulate else _out_type(dw)
    return (M, N, K, _ptr(qdyt), _ld(qdyt), _ptr(sdyt), _ld(sdyt), fdy, _ptr(qxt), _ld(qxt),
            _ptr(sxt), _ld(sxt), fx, _ptr(dw), ot, _ld(dw), wsp, wsb, _stream(dw))


def fp8bq_quantize_tensor_workspace_size(R, C):
    return int(lib().fp8bq_quantize_tensor_workspace_size(int(R), int(C)))


@_entry
def fp8bq_quantize_tensor_delayed(x, fmt, amax, beta, q, qt, s, ws):
    R, C = x.shape
    _expect_all([(x, "x", (R, C), _HI), (amax, "amax", (1,), _F32), (q, "q", (R, C), _U8),
                 (qt, "qt", (C, R), _U8), (s, "s", (1,), _F32)], ws)
    wsp, wsb = _ws_args(ws)
    return (_ptr(x), _in_type(x), R, C, _ld(x), fmt, _ptr(amax), float(beta), _ptr(q),
            _ld(q), _ptr(qt), _ld(qt) if qt is not None else 0, _ptr(s), wsp, wsb,
            _stream(x))


@_entry
def fp8bq_quantize_tensor_delayed_noalloc(x, fmt, amax, beta, q, qt, s):
    R, C = x.shape
    _expect_all([(x, "x", (R, C), _HI), (amax, "amax", (1,), _F32), (q, "q", (R, C), _U8),
                 (qt, "qt", (C, R), _U8), (s, "s", (1,), _F32)])
    return (_ptr(x), _in_type(x), R, C, _ld(x), fmt, _ptr(amax), float(beta),
            _ptr(q), _ld(q), _ptr(qt), _ld(qt) if qt is not None else 0,
            _ptr(s), _stream(x))


@_entry
def fp8bq_gemm_tensor(qa, sa, fa, qb, sb, fb, out, ws=None):
    M, K = qa.shape
    N = qb.shape[0]
    _expect_all([(qa, "qa", (M, K), _U8), (sa, "sa", (1,), _F32), (qb, "qb", (N, K), _U8), (sb, "sb", (1,), _F32),
                 (out, "out", (M, N), _HI)], ws)
    wsp, wsb = _ws_args(ws)
    return (M, N, K, _ptr(qa), _ld(qa), _ptr(sa), fa, _ptr(qb), _ld(qb), _ptr(sb), fb,
            _ptr(out), _out_type(out), _ld(out), wsp, wsb, _stream(out))


def fp8bq_hyperball_workspace_size(R, C):
    return int(lib().fp8bq_hyperball_workspace_size(int(R), int(C)))


@_entry
def fp8bq_hyperball_step(w, g, lr, weight_decay, eps, radius, norms, ws):
    R, C = w.shape
    _expect_all([(w, "w", (R, C), _F32), (g, "g", (R, C), _HI), (norms, "norms", (2,), _F32)], ws)
    wsp, wsb = _ws_args(ws)
    return (_ptr(w), _ld(w), _ptr(g), _in_type(g), _ld(g), R, C, float(lr),
            float(weight_decay), float(eps), float(radius), _ptr(norms), wsp, wsb,
            _stream(w))


@_entry
def fp8bq_stream_copy(src, dst):
    """Copy the bytes of contiguous tensor src into dst (same byte size): the streaming-copy
    bandwidth reference, not an operation of the layer."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous torch tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must hold the same number of bytes")
    if src.device.type != "cuda" or dst.device != src.device:
        raise ValueError("src and dst must be on the same CUDA (HIP) device")
    return (_ptr(src), _ptr(dst), nbytes, _stream(src))


def fp8bq_hyperball_batch_workspace_size(count):
    return int(lib().fp8bq_hyperball_batch_workspace_size(int(count)))


@_entry
def fp8bq_hyperball_step_batch(jobs, lr, weight_decay, eps, ws):
    """jobs: (w, g, radius, norms) per matrix, as fp8bq_hyperball_step takes them (norms None or a
    two-element FP32 tensor); every g of one dtype.  Two launches on the current stream of the first
    weight's device for all of them."""
    jobs = list(jobs)
    arr = (HyperballJob * max(len(jobs), 1))()
    gt = _in_type(jobs[0][1]) if jobs else IN_BF16
    if any(_in_type(job[1]) != gt for job in jobs):
        raise TypeError("all gradients of one fp8bq_hyperball_step_batch call must share one dtype")
    for i, (w, g, radius, norms) in enumerate(jobs):
        R, C = w.shape
        _expect_all([(jobs[0][0], "jobs[0].w", jobs[0][0].shape, _F32), (w, f"jobs[{i}].w", (R, C), _F32),
                     (g, f"jobs[{i}].g", (R, C), _HI), (norms, f"jobs[{i}].norms", (2,), _F32)], ws)
        arr[i] = HyperballJob(w.data_ptr(), _ld(w), g.data_ptr(), _ld(g), R, C, float(radius),
                              norms.data_ptr() if norms is not None else None)
    wsp, wsb = _ws_args(ws)
    stream = _stream(jobs[0][0]) if jobs else ctypes.c_void_p(0)
    return (arr, len(jobs), gt, float(lr), float(weight_decay), float(eps), wsp, wsb, stream)


# ---------------------------------------------------------------------------------------------
# allocating helpers
# ---------------------------------------------------------------------------------------------

def _pad4(n):
    return max(4, (n + 3) // 4 * 4)


def quantize_act_1x128(x, fmt=E4M3):
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    s = torch.empty((C // 128, _pad4(R)), dtype=torch.float32, device=x.device)[:, :R]
    fp8bq_quantize_act_1x128(x, fmt, q, s)
    return q, s


def quantize_act_128x1(x, fmt=E4M3):
    R, C = x.shape
    qt = torch.empty((C, R), dtype=torch.uint8, device=x.device)
    st = torch.empty((R // 128, _pad4(C)), dtype=torch.float32, device=x.device)[:, :C]
    fp8bq_quantize_act_128x1(x, fmt, qt, st)
    return qt, st


def quantize_act_dual(x, fmt_rows=E4M3, fmt_cols=E4M3):
    """(q, s) of quantize_act_1x128(x, fmt_rows) and (qt, st) of quantize_act_128x1(x, fmt_cols) from one
    pass over x (R and C multiples of 128)."""
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    s = torch.empty((C // 128, _pad4(R)), dtype=torch.float32, device=x.device)[:, :R]
    qt = torch.empty((C, R), dtype=torch.uint8, device=x.device)
    st = torch.empty((R // 128, _pad4(C)), dtype=torch.float32, device=x.device)[:, :C]
    fp8bq_quantize_act_dual(x, fmt_rows, q, s, fmt_cols, qt, st)
    return q, s, qt, st


def quantize_weight_dual(w, fmt=E4M3):
    """(q, s) of quantize_weight_128x128(w, fmt) and the transposed codes qt [K, N], one pass over w."""
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    qt = torch.empty((K, N), dtype=torch.uint8, device=w.device)
    fp8bq_quantize_weight_dual(w, fmt, q, s, qt)
    return q, s, qt


def quantize_weights_dual(ws, fmt=E4M3):
    """quantize_weight_dual of every weight in ws (all of one dtype), one launch per MAX_WEIGHT_JOBS weights."""
    outs = []
    for w in ws:
        N, K = w.shape
        outs.append((torch.empty((N, K), dtype=torch.uint8, device=w.device),
                     torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device),
                     torch.empty((K, N), dtype=torch.uint8, device=w.device)))
    ws = list(ws)
    for i in range(0, len(ws), MAX_WEIGHT_JOBS):
        fp8bq_quantize_weights_dual([(w,) + o for w, o in zip(ws[i:i + MAX_WEIGHT_JOBS], outs[i:i + MAX_WEIGHT_JOBS])],
                                    fmt)
    return outs


def quantize_weight_128x128(w, fmt=E4M3):
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    fp8bq_quantize_weight_128x128(w, fmt, q, s)
    return q, s


def _workspace(op, M, N, K, device):
    n = fp8bq_gemm_workspace_size(op, M, N, K)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def gemm_fprop(qx, sx, qw, sw, fx=E4M3, fw=E4M3, out_dtype=torch.bfloat16, out=None, ws=None):
    M, K = qx.shape
    N = qw.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=qx.device)
    if ws is None:
        ws = _workspace(OP_FPROP, M, N, K, qx.device)
    fp8bq_gemm_fprop(qx, sx, fx, qw, sw, fw, y, ws)
    return y


def gemm_dgrad(qdy, sdy, qw, sw, fdy=E4M3, fw=E4M3, out_dtype=torch.bfloat16, out=None, ws=None):
    M, N = qdy.shape
    K = qw.shape[1]
    dx = out if out is not None else torch.empty((M, K), dtype=out_dtype, device=qdy.device)
    if ws is None:
        ws = _workspace(OP_DGRAD, M, N, K, qdy.device)
    fp8bq_gemm_dgrad(qdy, sdy, fdy, qw, sw, fw, dx, ws)
    return dx


def gemm_dgrad_wt(qdy, sdy, qwt, sw, fdy=E4M3, fw=E4M3, out_dtype=torch.bfloat16, out=None, ws=None):
    M, N = qdy.shape
    K = qwt.shape[0]
    dx = out if out is not None else torch.empty((M, K), dtype=out_dtype, device=qdy.device)
    if ws is None:
        ws = _workspace(OP_DGRAD_WT, M, N, K, qdy.device)
    fp8bq_gemm_dgrad_wt(qdy, sdy, fdy, qwt, sw, fw, dx, ws)
    return dx


def gemm_wgrad(qdyt, sdyt, qxt, sxt, fdy=E4M3, fx=E4M3, out_dtype=torch.bfloat16, out=None, ws=None,
               accumulate=False):
    """accumulate=True adds the result to `out` (an FP32 main-grad buffer) instead of overwriting it."""
    N, M = qdyt.shape
    K = qxt.shape[0]
    if accumulate and (out is None or out.dtype != torch.float32):
        raise ValueError("accumulate=True needs an FP32 `out` tensor holding the running sum")
    dw = out if out is not None else torch.empty((N, K), dtype=out_dtype, device=qdyt.device)
    if ws is None:
        ws = _workspace(OP_WGRAD, M, N, K, qdyt.device)
    fp8bq_gemm_wgrad(qdyt, sdyt, fdy, qxt, sxt, fx, dw, ws, accumulate=accumulate)
    return dw


def quantize_tensor_delayed(x, amax, beta=0.99, fmt=E4M3, transpose=False):
    """Per-tensor delayed scaling: updates the one-element FP32 running amax `amax` in place with
    max|x| and returns (q [R, C] codes of x's BF16 copy, s (one-element FP32 scale), qt [C, R] or None)."""
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    qt = torch.empty((C, R), dtype=torch.uint8, device=x.device) if transpose else None
    s = torch.empty(1, dtype=torch.float32, device=x.device)
    n = fp8bq_quantize_tensor_workspace_size(R, C)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=x.device)
    fp8bq_quantize_tensor_delayed(x, fmt, amax, beta, q, qt, s, ws)
    return q, s, qt


def gemm_tensor(qa, sa, qb, sb, fa=E4M3, fb=E4M3, out_dtype=torch.bfloat16, out=None, ws=None):
    """out [M, N] = sa * sb * dec(qa) . dec(qb)^T for per-tensor scales sa, sb (one-element tensors)."""
    M, K = qa.shape
    N = qb.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=qa.device)
    if ws is None:
        ws = _workspace(OP_TENSOR, M, N, K, qa.device)
    fp8bq_gemm_tensor(qa, sa, fa, qb, sb, fb, y, ws)
    return y


def hyperball_step(w, g, lr=1e-4, weight_decay=0.1, eps=1e-8, radius=0.0, ws=None):
    """In-place Hyperball update of the FP32 weight w with gradient g (BF16 or FP32); returns a
    two-element FP32 device tensor (||g||, ||w|| after the update and before the projection)."""
    if w.dtype != torch.float32:
        raise TypeError("w must be the FP32 master weight")
    if w.shape != g.shape:
        raise ValueError("w and g must have one shape")
    norms = torch.empty(2, dtype=torch.float32, device=w.device)
    if ws is None:
        ws = torch.empty(max(fp8bq_hyperball_workspace_size(*w.shape), 16), dtype=torch.uint8, device=w.device)
    fp8bq_hyperball_step(w, g, lr, weight_decay, eps, radius, norms, ws)
    return norms


def hyperball_step_batch(weights, grads, lr=1e-4, weight_decay=0.1, eps=1e-8, radii=None, ws=None):
    """In-place Hyperball updates of many FP32 weights, MAX_HYPERBALL_JOBS per launch pair; grads
    of one dtype; radii: None (no projection) or one radius per weight.  Returns an [n, 2] FP32
    device tensor of (||g||, ||w|| after the update and before the projection) per weight."""
    weights, grads = list(weights), list(grads)
    if len(weights) != len(grads):
        raise ValueError("one gradient per weight")
    radii = [0.0] * len(weights) if radii is None else [float(r) for r in radii]
    if len(radii) != len(weights):
        raise ValueError("one radius per weight")
    if not weights:
        return torch.empty((0, 2), dtype=torch.float32)
    dev = weights[0].device
    norms = torch.empty((len(weights), 2), dtype=torch.float32, device=dev)
    n = min(len(weights), MAX_HYPERBALL_JOBS)
    if ws is None:
        ws = torch.empty(fp8bq_hyperball_batch_workspace_size(n), dtype=torch.uint8, device=dev)
    for i in range(0, len(weights), MAX_HYPERBALL_JOBS):
        sl = slice(i, i + MAX_HYPERBALL_JOBS)
        fp8bq_hyperball_step_batch([(w, g, r, norms[k]) for k, (w, g, r) in
                                    zip(range(i, i + MAX_HYPERBALL_JOBS), zip(weights[sl], grads[sl], radii[sl]))],
                                   lr, weight_decay, eps, ws)
    return norms
