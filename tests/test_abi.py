"""C-ABI checks that need no GPU: the library loads, exports every function include/fp8bq.h
declares, and rejects bad arguments with the documented status before touching the device.

Pointers passed here are fake (16-byte aligned integers); every call is expected to return during
argument validation, or with FP8BQ_ERR_DEVICE on a machine without a gfx950 GPU.
"""

import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch

import fp8_blockwise_quantized_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bq.h")

OK, NULL, SHAPE, LD, ALIGN, DTYPE, FORMAT, WORKSPACE, DEVICE, LAUNCH, OVERLAP, VALUE = range(12)
HAVE_GPU = torch.cuda.is_available()

P = lambda i: ctypes.c_void_p(0x100000 * (i + 1))  # disjoint, 16-byte aligned fake buffers
NUL = ctypes.c_void_p(0)
S0 = ctypes.c_void_p(0)  # stream


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8bq_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = fq.lib()
    names = declared_functions()
    assert len(names) == 23, names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert fq.lib().fp8bq_version() >= 100
    for st in range(12):
        s = fq.status_string(st)
        assert s.startswith("FP8BQ_")
    assert fq.status_string(4242) == "FP8BQ_ERR_UNKNOWN"


def q1x128(x=P(0), xt=0, R=256, C=256, ldx=256, fmt=0, q=P(1), ldq=256, s=P(2), lds=256):
    return fq.lib().fp8bq_quantize_act_1x128(x, xt, R, C, ldx, fmt, q, ldq, s, lds, S0)


def q128x1(x=P(0), xt=0, R=256, C=64, ldx=64, fmt=0, qt=P(1), ldqt=256, st=P(2), ldst=64):
    return fq.lib().fp8bq_quantize_act_128x1(x, xt, R, C, ldx, fmt, qt, ldqt, st, ldst, S0)


def qw(w=P(0), wt=0, N=256, K=256, ldw=256, fmt=0, q=P(1), ldq=256, s=P(2), lds=2):
    return fq.lib().fp8bq_quantize_weight_128x128(w, wt, N, K, ldw, fmt, q, ldq, s, lds, S0)


def valid(call):
    """A call with valid arguments passes validation and stops at the device check on a machine
    without a gfx950 GPU.  On a GPU machine it would launch kernels on the fake pointers, so it is
    not made there."""
    if not HAVE_GPU:
        assert call() == DEVICE


@pytest.mark.skipif(HAVE_GPU, reason="checks the no-device path")
def test_valid_arguments_reach_the_device_check():
    assert q1x128() == DEVICE
    assert q128x1() == DEVICE
    assert qw() == DEVICE
    assert qw(lds=3) == DEVICE  # weight scales need no ld alignment
    assert qdual() == DEVICE
    assert qwdual() == DEVICE
    assert gemm("fp8bq_gemm_dgrad_wt", ws=NUL, ws_bytes=0) == DEVICE  # no transpose: no workspace


def test_quant_1x128_validation():
    assert q1x128(xt=7) == DTYPE
    assert q1x128(fmt=2) == FORMAT
    assert q1x128(C=200, ldx=200, ldq=208) == SHAPE
    assert q1x128(R=-1) == SHAPE
    assert q1x128(R=0, x=NUL, q=NUL, s=NUL) == OK  # empty: no-op
    assert q1x128(x=NUL) == NULL
    assert q1x128(s=NUL) == NULL
    assert q1x128(x=ctypes.c_void_p(0x100008)) == ALIGN
    assert q1x128(ldx=128) == LD
    assert q1x128(ldx=260) == LD  # 520 bytes, not a multiple of 16
    assert q1x128(ldq=264) == LD
    assert q1x128(lds=255) == LD
    assert q1x128(lds=258) == LD  # scales: ld % 4
    assert q1x128(q=P(0)) == OVERLAP


def test_quant_128x1_validation():
    assert q128x1(R=200) == SHAPE
    assert q128x1(C=12, ldx=16, ldst=16) == SHAPE  # C % 8
    assert q128x1(ldqt=128) == LD
    assert q128x1(ldst=60) == LD
    assert q128x1(C=0) == OK
    assert q128x1(st=P(0)) == OVERLAP


def test_quant_weight_validation():
    assert qw(N=200) == SHAPE
    assert qw(K=100, ldw=112, ldq=112) == SHAPE
    assert qw(lds=1) == LD
    assert qw(wt=1, ldw=254) == LD


def gemm(fn, M=256, N=256, K=256, qa=P(0), ldqa=256, sa=P(1), ldsa=256, fa=0, qb=P(2), ldqb=256, sb=P(3), ldsb=2,
         fb=0, out=P(4), out_t=0, ldout=256, ws=P(5), ws_bytes=1 << 20):
    return getattr(fq.lib(), fn)(M, N, K, qa, ldqa, sa, ldsa, fa, qb, ldqb, sb, ldsb, fb, out, out_t, ldout, ws,
                                 ws_bytes, S0)


def test_gemm_validation():
    for fn in ("fp8bq_gemm_fprop", "fp8bq_gemm_dgrad"):
        valid(lambda: gemm(fn))
        assert gemm(fn, K=200) == SHAPE
        assert gemm(fn, N=200) == SHAPE
        valid(lambda: gemm(fn, M=100, ldsa=100))  # ragged token count is allowed
        assert gemm(fn, fa=3) == FORMAT
        assert gemm(fn, out_t=5) == DTYPE
        assert gemm(fn, qa=NUL) == NULL
        assert gemm(fn, out=NUL) == NULL
        assert gemm(fn, ldout=100) == LD
        assert gemm(fn, ldsa=250) == LD
        assert gemm(fn, out=P(0)) == OVERLAP
        assert gemm(fn, M=0, qa=NUL, out=NUL) == OK
        assert gemm(fn, out_t=2) == DTYPE  # FP32 accumulation is a wgrad option only
    assert gemm("fp8bq_gemm_dgrad_wt", out_t=2, ws=NUL, ws_bytes=0) == DTYPE
    w = "fp8bq_gemm_wgrad"
    valid(lambda: gemm(w, ldsb=256))
    valid(lambda: gemm(w, ldsb=256, out_t=2))
    assert gemm(w, ldsb=256, out_t=3) == DTYPE
    valid(lambda: gemm(w, M=0, qa=NUL, sa=NUL, qb=NUL, sb=NUL, ldsb=256, out_t=2))  # an empty sum
    assert gemm(w, M=200, ldqa=208, ldqb=208, ldsb=256) == SHAPE  # contraction must be a multiple of 128
    assert gemm(w, ldsb=2) == LD  # column scales are read as vectors
    # a 256-row tile of codes is addressed through a 32-bit range: 2^24 tokens is one too many rows
    big = 1 << 24
    assert gemm(w, M=big, ldqa=big, ldqb=big, ldsa=256, ldsb=256) == LD
    far = lambda i: ctypes.c_void_p((i + 1) << 36)  # fake buffers 64 GiB apart
    valid(lambda: gemm(w, M=big - 128, ldqa=big - 128, ldqb=big - 128, ldsb=256, qa=far(0), sa=far(1), qb=far(2),
                       sb=far(3), out=far(4), ws=far(5), ws_bytes=1 << 34))
    assert gemm("fp8bq_gemm_fprop", ldqa=(1 << 32) // 255) == LD
    # dgrad needs a workspace for the transposed weight codes
    need = fq.fp8bq_gemm_workspace_size(fq.OP_DGRAD, 256, 256, 256)
    assert need >= 256 * 256
    assert gemm("fp8bq_gemm_dgrad", ws=NUL, ws_bytes=0) == WORKSPACE
    assert gemm("fp8bq_gemm_dgrad", ws_bytes=need - 1) == WORKSPACE
    assert gemm("fp8bq_gemm_dgrad", ws=ctypes.c_void_p(0x600008)) == ALIGN


def test_workspace_sizes():
    assert fq.fp8bq_gemm_workspace_size(fq.OP_FPROP, 8192, 8192, 2048) >= 0
    assert fq.fp8bq_gemm_workspace_size(fq.OP_DGRAD, 16384, 11264, 2048) >= 11264 * 2048
    assert fq.fp8bq_gemm_workspace_size(7, 1, 1, 1) == 0
    assert fq.fp8bq_gemm_workspace_size(fq.OP_WGRAD, -1, 1, 1) == 0


def test_zero_contraction_is_valid():
    # K == 0 makes Y all zeros: only the output must be valid
    valid(lambda: gemm("fp8bq_gemm_fprop", K=0, qa=NUL, sa=NUL, qb=NUL, sb=NUL))


def test_gemm_plan_query():
    """The plan query validates its arguments and reports one of the built tile shapes; the
    workspace size agrees with the split it reports (FP32 partials of split x rows x cols)."""
    lib = fq.lib()
    i32 = ctypes.c_int32
    a, b, c = i32(-1), i32(-1), i32(-1)
    ref = lambda v: ctypes.cast(ctypes.byref(v), ctypes.c_void_p)
    assert lib.fp8bq_gemm_plan(0, 256, 256, 256, NUL, ref(b), ref(c)) == NULL
    assert lib.fp8bq_gemm_plan(5, 256, 256, 256, ref(a), ref(b), ref(c)) == SHAPE
    assert lib.fp8bq_gemm_plan(0, -1, 256, 256, ref(a), ref(b), ref(c)) == SHAPE
    assert a.value == -1 and b.value == -1 and c.value == -1
    for op in (fq.OP_FPROP, fq.OP_DGRAD, fq.OP_WGRAD, fq.OP_DGRAD_WT, fq.OP_TENSOR):
        for (M, N, K) in [(256, 256, 256), (512, 2048, 2048), (16384, 2560, 2048), (16384, 11264, 2048),
                          (16384, 2048, 5632)]:
            tm, tn, sk = fq.fp8bq_gemm_plan(op, M, N, K)
            assert (tm, tn) in [(64, 64), (128, 128), (256, 256)]
            assert 1 <= sk <= 8
            rows, cols = {fq.OP_FPROP: (M, N), fq.OP_DGRAD: (M, K), fq.OP_WGRAD: (N, K), fq.OP_DGRAD_WT: (M, K),
                          fq.OP_TENSOR: (M, N)}[op]
            ws = fq.fp8bq_gemm_workspace_size(op, M, N, K)
            transpose = ((N * K + 255) // 256) * 256 if op == fq.OP_DGRAD else 0
            assert ws == transpose + (sk * rows * cols * 4 if sk > 1 else 0)


def qdual(x=P(0), xt=0, R=256, C=256, ldx=256, fr=0, q=P(1), ldq=256, s=P(2), lds=256, fc=0, qt=P(3), ldqt=256,
          st=P(4), ldst=256):
    return fq.lib().fp8bq_quantize_act_dual(x, xt, R, C, ldx, fr, q, ldq, s, lds, fc, qt, ldqt, st, ldst, S0)


def test_quant_dual_validation():
    assert qdual(R=0) == OK and qdual(C=0) == OK  # empty: no-op
    assert qdual(xt=2) == DTYPE
    assert qdual(fr=2) == FORMAT and qdual(fc=-1) == FORMAT
    assert qdual(R=200) == SHAPE  # 128x1 groups need R % 128 == 0
    assert qdual(C=200, ldx=256) == SHAPE  # 1x128 groups need C % 128 == 0
    assert qdual(q=NUL) == NULL and qdual(st=NUL) == NULL
    assert qdual(ldqt=200) == LD and qdual(lds=250) == LD
    assert qdual(qt=P(1)) == OVERLAP  # the two code arrays coincide
    assert qdual(st=P(2)) == OVERLAP
    assert qdual(s=P(0)) == OVERLAP  # scales on top of the input


def qwdual(w=P(0), wt=0, N=256, K=256, ldw=256, fmt=0, q=P(1), ldq=256, s=P(2), lds=2, qt=P(3), ldqt=256):
    return fq.lib().fp8bq_quantize_weight_dual(w, wt, N, K, ldw, fmt, q, ldq, s, lds, qt, ldqt, S0)


def test_quant_weight_dual_validation():
    assert qwdual(N=0) == OK
    assert qwdual(wt=3) == DTYPE and qwdual(fmt=5) == FORMAT
    assert qwdual(N=200) == SHAPE and qwdual(K=100, ldw=112, ldq=112) == SHAPE
    assert qwdual(qt=NUL) == NULL
    assert qwdual(ldqt=200) == LD  # ldqt >= N
    assert qwdual(ldqt=264) == LD  # 16-byte rows
    assert qwdual(qt=P(1)) == OVERLAP and qwdual(qt=P(0)) == OVERLAP


def wjob(base, N=256, K=256, ldw=256, ldq=256, lds=2, ldqt=256, w=None, q=None, s=None, qt=None):
    """A fake weight job whose four buffers sit at P(base) .. P(base + 3) unless given."""
    pick = lambda v, i: (v if v is not None else P(base + i)).value or 0
    return fq.WeightJob(pick(w, 0), N, K, ldw, pick(q, 1), ldq, pick(s, 2), lds, pick(qt, 3), ldqt)


def qwbatch(jobs, wt=0, fmt=0, count=None):
    arr = (fq.WeightJob * max(len(jobs), 1))(*jobs)
    return fq.lib().fp8bq_quantize_weights_dual(arr, len(jobs) if count is None else count, wt, fmt, S0)


def test_quant_weights_batch_validation():
    lib = fq.lib()
    assert lib.fp8bq_quantize_weights_dual(None, 0, 0, 0, S0) == OK  # nothing to do
    assert lib.fp8bq_quantize_weights_dual(None, 2, 0, 0, S0) == NULL
    assert qwbatch([wjob(0)], count=-1) == VALUE and qwbatch([wjob(0)], count=17) == VALUE
    assert qwbatch([wjob(0, N=0), wjob(4, K=0)]) == OK  # only empty jobs: nothing enqueued
    valid(lambda: qwbatch([wjob(0), wjob(4, N=384, K=128, ldw=128, ldq=128, lds=4, ldqt=384)]))
    valid(lambda: qwbatch([wjob(4 * i) for i in range(16)]))
    # each job gets the single-weight checks, in job order
    assert qwbatch([wjob(0)], wt=3) == DTYPE and qwbatch([wjob(0)], fmt=5) == FORMAT
    assert qwbatch([wjob(0), wjob(4, N=200)]) == SHAPE
    assert qwbatch([wjob(0), wjob(4, qt=NUL)]) == NULL
    assert qwbatch([wjob(0), wjob(4, ldqt=200)]) == LD
    assert qwbatch([wjob(0), wjob(4, qt=P(5))]) == OVERLAP  # within one job
    # across jobs: outputs may not touch another job's input or outputs; inputs may be shared
    assert qwbatch([wjob(0), wjob(4, q=P(0))]) == OVERLAP  # job 1's codes over job 0's weight
    assert qwbatch([wjob(0), wjob(4, qt=P(1))]) == OVERLAP  # job 1's W^T codes over job 0's codes
    assert qwbatch([wjob(0), wjob(4, s=P(3))]) == OVERLAP  # job 1's scales in job 0's W^T codes
    assert qwbatch([wjob(0, q=P(6)), wjob(4)]) == OVERLAP  # job 0's codes over job 1's scales
    valid(lambda: qwbatch([wjob(0), wjob(4, w=P(0))]))  # both read one weight
    valid(lambda: qwbatch([wjob(0), wjob(4, q=P(0), N=0)]))  # an empty job's buffers are never touched
    # the tiles of all jobs together must fit one grid: 2^16 x 2^15 tiles in one (fake, disjoint) job
    N, K = 1 << 23, 1 << 22
    far = lambda e: ctypes.c_void_p(1 << e)
    big = wjob(0, N=N, K=K, ldw=K, ldq=K, lds=K // 128, ldqt=N, w=far(47), q=far(48), s=far(49), qt=far(50))
    assert qwbatch([big]) == SHAPE


def test_gemm_dgrad_wt_validation():
    g = "fp8bq_gemm_dgrad_wt"
    assert gemm(g, K=200) == SHAPE and gemm(g, N=200) == SHAPE
    assert gemm(g, qb=NUL) == NULL
    assert gemm(g, out=P(2)) == OVERLAP
    assert gemm(g, ldqb=100) == LD  # W^T rows hold N codes
    assert fq.fp8bq_gemm_workspace_size(fq.OP_DGRAD_WT, 16384, 11264, 2048) < 11264 * 2048  # no transpose buffer


def qtensor(x=P(0), xt=0, R=256, C=256, ldx=256, fmt=0, amax=P(1), beta=0.99, q=P(2), ldq=256, qt=P(3), ldqt=256,
            s=ctypes.c_void_p(0x100000 * 2 + 64), ws=P(4), ws_bytes=8192):
    return fq.lib().fp8bq_quantize_tensor_delayed(x, xt, R, C, ldx, fmt, amax, beta, q, ldq, qt, ldqt, s, ws, ws_bytes,
                                                  S0)


def test_quant_tensor_delayed_validation():
    assert 4096 < fq.fp8bq_quantize_tensor_workspace_size(256, 256) <= 8192
    assert fq.fp8bq_quantize_tensor_workspace_size(0, 256) == 0
    valid(lambda: qtensor(s=P(5)))
    valid(lambda: qtensor(s=P(5), qt=NUL, R=200))  # ragged rows without the transposed codes
    assert qtensor(R=0) == OK and qtensor(C=0) == OK  # empty: nothing enqueued
    assert qtensor(xt=2) == DTYPE and qtensor(fmt=2) == FORMAT
    assert qtensor(beta=1.5) == VALUE and qtensor(beta=-0.01) == VALUE and qtensor(beta=float("nan")) == VALUE
    valid(lambda: qtensor(s=P(5), beta=0.0))
    valid(lambda: qtensor(s=P(5), beta=1.0))
    assert qtensor(C=200, ldx=256) == SHAPE
    assert qtensor(R=200) == SHAPE  # the transposed codes need R % 128 == 0
    assert qtensor(amax=NUL) == NULL and qtensor(ws=NUL) == NULL and qtensor(q=NUL) == NULL
    assert qtensor(amax=ctypes.c_void_p(0x200002)) == ALIGN
    assert qtensor(ws_bytes=100) == WORKSPACE
    assert qtensor(ldq=100) == LD and qtensor(ldqt=100) == LD
    assert qtensor(q=P(0)) == OVERLAP  # codes over the input
    assert qtensor(s=P(1)) == OVERLAP  # scale and running amax in one float
    assert qtensor(s=P(5), amax=P(4)) == OVERLAP  # running amax inside the workspace


def test_gemm_tensor_validation():
    def gt(M=256, N=256, K=256, qa=P(0), ldqa=256, sa=P(1), fa=0, qb=P(2), ldqb=256, sb=P(3), fb=0, out=P(4),
           out_t=0, ldout=256, ws=P(5), ws_bytes=1 << 20):
        return fq.lib().fp8bq_gemm_tensor(M, N, K, qa, ldqa, sa, fa, qb, ldqb, sb, fb, out, out_t, ldout, ws,
                                          ws_bytes, S0)
    valid(lambda: gt())
    valid(lambda: gt(M=100, sa=ctypes.c_void_p(0x200004)))  # ragged rows; a scale needs 4-byte alignment only
    assert gt(sa=ctypes.c_void_p(0x200002)) == ALIGN
    assert gt(K=200) == SHAPE and gt(N=200) == SHAPE
    assert gt(sb=NUL) == NULL and gt(fb=4) == FORMAT and gt(out_t=2) == DTYPE
    assert gt(out=P(0)) == OVERLAP
    assert gt(M=0, qa=NUL, out=NUL) == OK
    assert fq.fp8bq_gemm_plan(fq.OP_TENSOR, 4096, 2048, 2048) == fq.fp8bq_gemm_plan(fq.OP_FPROP, 4096, 2048, 2048)


def hb(w=P(0), ldw=256, g=P(1), gt=0, ldg=256, R=256, C=256, lr=1e-4, wd=0.1, eps=1e-8, radius=0.0, norms=P(2),
       ws=P(3), ws_bytes=1 << 16):
    return fq.lib().fp8bq_hyperball_step(w, ldw, g, gt, ldg, R, C, lr, wd, eps, radius, norms, ws, ws_bytes, S0)


def test_stream_copy_validation():
    c = lambda src=P(0), dst=P(1), n=4096: fq.lib().fp8bq_stream_copy(src, dst, n, S0)
    assert c(n=0) == OK and c(src=NUL, dst=NUL, n=0) == OK  # empty: a no-op, pointers unread
    assert c(n=100) == SHAPE
    assert c(n=1 << 48) == SHAPE
    assert c(src=NUL) == NULL and c(dst=NUL) == NULL
    assert c(src=ctypes.c_void_p(0x100008)) == ALIGN
    assert c(dst=ctypes.c_void_p(0x100000 + 2048)) == OVERLAP  # dst starts inside src's 4096 bytes
    assert c(src=ctypes.c_void_p(0x200000 - 2048)) == OVERLAP  # src ends inside dst
    valid(lambda: c())
    valid(lambda: c(src=ctypes.c_void_p(0x200000 - 4096)))  # adjacent ranges are fine


def test_hyperball_validation():
    need = fq.fp8bq_hyperball_workspace_size(256, 256)
    assert 16 * 1024 <= need <= 1 << 16 and fq.fp8bq_hyperball_workspace_size(0, 8) == 0
    valid(lambda: hb())
    valid(lambda: hb(norms=NUL, radius=3.0, C=264, ldw=264, ldg=264, R=7))
    assert hb(R=0) == OK
    assert hb(gt=2) == DTYPE
    assert hb(C=100, ldw=256, ldg=256) == SHAPE
    for bad in (dict(lr=-1.0), dict(wd=-0.1), dict(eps=0.0), dict(eps=float("inf")), dict(radius=-2.0),
                dict(lr=float("nan")), dict(radius=float("inf"))):
        assert hb(**bad) == VALUE, bad
    assert hb(w=NUL) == NULL and hb(ws=NUL) == NULL
    assert hb(ldw=100) == LD and hb(ldg=250) == LD
    assert hb(norms=ctypes.c_void_p(0x300002)) == ALIGN
    assert hb(ws_bytes=need - 1) == WORKSPACE
    assert hb(g=P(0)) == OVERLAP  # gradient on top of the weights
    assert hb(norms=ctypes.c_void_p(0x100000 + 64)) == OVERLAP  # norms inside w


def hbb(jobs, count=None, gt=0, lr=1e-4, wd=0.1, eps=1e-8, ws=P(9), ws_bytes=None):
    """fp8bq_hyperball_step_batch on fake pointers; jobs: dicts of HyperballJob fields."""
    n = len(jobs) if count is None else count
    arr = (fq.HyperballJob * max(len(jobs), 1))()
    for i, j in enumerate(jobs):
        arr[i] = fq.HyperballJob(**j)
    need = fq.fp8bq_hyperball_batch_workspace_size(max(n, 0))
    return fq.lib().fp8bq_hyperball_step_batch(arr, n, gt, lr, wd, eps, ws, need if ws_bytes is None else ws_bytes, S0)


def hbjob(i, R=256, C=256, radius=0.0, norms=None):
    """Job i on fake buffers 0x100000 * (2i + 1) (w) and 0x100000 * (2i + 2) (g)."""
    return dict(w=0x100000 * (2 * i + 1), ldw=C, g=0x100000 * (2 * i + 2), ldg=C, R=R, C=C, radius=radius,
                norms=norms)


def test_hyperball_batch_validation():
    assert fq.fp8bq_hyperball_batch_workspace_size(4) == 4 * fq.fp8bq_hyperball_workspace_size(256, 256)
    assert fq.fp8bq_hyperball_batch_workspace_size(33) == 0 and fq.fp8bq_hyperball_batch_workspace_size(-1) == 0
    two = [hbjob(0), hbjob(1, R=7, C=264, radius=2.0, norms=0x10000000)]
    valid(lambda: hbb(two))
    assert hbb([]) == OK and hbb([hbjob(0, R=0), hbjob(1, C=0)], ws=NUL) == OK  # nothing to do: ws unread
    assert hbb(two, count=33) == VALUE and hbb(two, count=-1) == VALUE
    assert fq.lib().fp8bq_hyperball_step_batch(None, 2, 0, 1e-4, 0.1, 1e-8, P(9), 1 << 20, S0) == NULL
    assert hbb(two, gt=2) == DTYPE
    assert hbb(two, eps=0.0) == VALUE and hbb([hbjob(0), hbjob(1, radius=-1.0)]) == VALUE
    assert hbb([hbjob(0), hbjob(1, C=100)]) == SHAPE  # the second job's error
    assert hbb(two, ws=NUL) == NULL and hbb(two, ws_bytes=1024) == WORKSPACE
    assert hbb(two, ws=ctypes.c_void_p(0x900008)) == ALIGN
    # one job's weights on top of another job's gradient, weights or norms; norms inside the workspace
    assert hbb([hbjob(0), dict(hbjob(1), w=0x100000 * 2)]) == OVERLAP
    assert hbb([hbjob(0), dict(hbjob(1), w=0x100000 * 1)]) == OVERLAP
    assert hbb([hbjob(0, norms=0x10000000), dict(hbjob(1), w=0x10000000 - 64)]) == OVERLAP
    assert hbb([hbjob(0, norms=0xA00000 + 64), hbjob(1)]) == OVERLAP  # the workspace is P(9) = 0xA00000
    # two jobs may read one gradient
    valid(lambda: hbb([hbjob(0), dict(hbjob(1), g=0x100000 * 2)]))


def test_planner_decisions_documented_for_the_decoder_block():
    """Plans the design records (device of 256 compute units; no GPU here, or an MI355X): the step's
    fprop/dgrad on 256x256 tiles unsplit (the QKV fprop's half-filled last round is charged half a
    round, which moves it off 128x128); small-token fprops are not split (the reduction pass costs a
    fixed launch) and take 64x64 tiles up to 1024 tokens; long-contraction wgrads with few output
    tiles are split."""
    if HAVE_GPU and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("plans are recorded for 256 compute units")
    M = 16384
    for K, N in [(2048, 2560), (2048, 2048), (2048, 11264), (5632, 2048)]:
        assert fq.fp8bq_gemm_plan(fq.OP_FPROP, M, N, K) == (256, 256, 1), (K, N)
        assert fq.fp8bq_gemm_plan(fq.OP_DGRAD_WT, M, N, K) == (256, 256, 1), (K, N)
    assert fq.fp8bq_gemm_plan(fq.OP_WGRAD, M, 2560, 2048) == (256, 256, 3)
    assert fq.fp8bq_gemm_plan(fq.OP_WGRAD, M, 2048, 2048) == (128, 128, 2)
    # token sweep (N = K = 2048): 64x64 tiles while 128x128 ones would leave most CUs idle
    for tokens, plan in ((512, (64, 64, 1)), (1024, (64, 64, 1)), (2048, (128, 128, 1)), (4096, (128, 128, 1)),
                         (8192, (256, 256, 1))):
        assert fq.fp8bq_gemm_plan(fq.OP_FPROP, tokens, 2048, 2048) == plan, tokens
    # the kernel forms the GPU format-pair tests run (64x64 and 128x128 tiles, whole and split; 256x256)
    forms = {fq.OP_FPROP: [((256, 384, 256), (64, 64, 1)), ((256, 256, 3072), (64, 64, 6)),
                           ((1024, 4096, 1024), (128, 128, 1)), ((128, 4096, 4096), (128, 128, 4)),
                           ((4096, 4096, 256), (256, 256, 1))],
             fq.OP_DGRAD: [((256, 384, 256), (64, 64, 1)), ((256, 3072, 256), (64, 64, 6)),
                           ((1024, 1024, 4096), (128, 128, 1)), ((128, 4096, 4096), (128, 128, 4)),
                           ((8192, 256, 2048), (256, 256, 1))],
             fq.OP_WGRAD: [((256, 384, 256), (64, 64, 1)), ((3072, 256, 256), (64, 64, 6)),
                           ((1024, 1024, 4096), (128, 128, 1)), ((4096, 128, 4096), (128, 128, 4)),
                           ((2048, 4096, 4096), (256, 256, 1))]}
    for op, cases in forms.items():
        for shape, plan in cases:
            assert fq.fp8bq_gemm_plan(op, *shape) == plan, (op, shape)
    # the plan is a pure function of its arguments
    assert all(fq.fp8bq_gemm_plan(fq.OP_WGRAD, 8192, 4096, 1024) == fq.fp8bq_gemm_plan(fq.OP_WGRAD, 8192, 4096, 1024)
               for _ in range(3))


@pytest.mark.skipif(shutil.which("gcc") is None or HAVE_GPU, reason="needs gcc; checks the no-device paths")
def test_c99_caller(tmp_path):
    """The header alone is a C99 interface: a C program (tests/csrc/abi_from_c.c) built with gcc
    -std=c99 -pedantic links against the library and gets the documented status codes, plans and
    workspace sizes without any HIP header."""
    src = os.path.join(ROOT, "tests", "csrc", "abi_from_c.c")
    libdir = os.path.dirname(fq.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    src, "-L", libdir, "-lfp8bq", f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr


def test_weights_batch_binding_rejects_mixed_dtypes_and_devices():
    """The binding's own checks, before the library is called (CPU tensors: no launch happens)."""
    w1 = torch.zeros((128, 128), dtype=torch.bfloat16)
    w2 = torch.zeros((128, 128), dtype=torch.float32)
    out = lambda: (torch.empty((128, 128), dtype=torch.uint8), torch.empty((1, 1), dtype=torch.float32),
                   torch.empty((128, 128), dtype=torch.uint8))
    with pytest.raises(TypeError):
        fq.fp8bq_quantize_weights_dual([(w1,) + out(), (w2,) + out()], fq.E4M3)
    q, s, qt = out()
    with pytest.raises(ValueError):
        fq.fp8bq_quantize_weights_dual([(w1, q, s, qt.to("meta"))], fq.E4M3)


def test_matrices_beyond_the_address_space_are_rejected():
    """A matrix whose byte extent reaches 2^48 cannot exist on the device; the check also keeps the
    overlap arithmetic free of overflow."""
    assert q1x128(R=1 << 41) == SHAPE  # 2^41 rows of 512 bytes
    assert q1x128(R=2, ldx=1 << 47) == SHAPE  # two rows 2^48 bytes apart
    assert q1x128(R=1 << 62, ldx=1 << 62) == SHAPE  # the product would overflow 64 bits
    valid(lambda: q1x128(R=1 << 20, ldx=1 << 20, q=P(1 << 22), ldq=256, s=P(1 << 23), lds=1 << 20))


def test_gemm_too_large_for_one_launch_is_refused():
    """2^22 x 2^22 outputs are 2^30 tiles of 128x128, more than one launch addresses: FP8BQ_ERR_SHAPE
    from the call and from fp8bq_gemm_plan, with buffers placed far apart so that no other check
    fires first."""
    M = N = 1 << 22
    far = lambda e: ctypes.c_void_p(1 << e)
    st = gemm("fp8bq_gemm_fprop", M=M, N=N, K=128, qa=far(40), ldqa=128, sa=far(41), ldsa=M, qb=far(42), ldqb=128,
              sb=far(43), ldsb=1, out=far(45), ldout=N, ws=far(44), ws_bytes=1 << 20)
    assert st == SHAPE
    tm, tn, sk = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    assert fq.lib().fp8bq_gemm_plan(fq.OP_FPROP, M, N, 128, ctypes.byref(tm), ctypes.byref(tn),
                                    ctypes.byref(sk)) == SHAPE
    assert fq.fp8bq_gemm_workspace_size(fq.OP_FPROP, M, N, 128) == 0


def test_host_code_under_sanitizers():
    """The validation and the planner (pure host C++) built with g++ and the address and
    undefined-behaviour sanitizers, driven by tests/csrc/host_checks.cpp over random and extreme
    arguments: no undefined behaviour, only documented statuses, consistent plans."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    csrc = os.path.join(ROOT, "fp8_blockwise_quantized_amd", "csrc")
    exe = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"fp8bq_host_checks_{os.getpid()}")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", csrc,
           os.path.join(ROOT, "tests", "csrc", "host_checks.cpp"), os.path.join(csrc, "validate.cpp"),
           os.path.join(csrc, "plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    finally:
        os.remove(exe)
