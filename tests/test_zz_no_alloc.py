"""The allocation-free entry point fp8bq_quantize_tensor_delayed_noalloc (the library's own scratch
in place of a caller workspace) against fp8bq_quantize_tensor_delayed, called through the C ABI:
running amax, scale, codes and transposed codes bit-identical, over two calls in a row whose second
input is smaller (the scratch keeps the first call's partial maxima), for BF16 and FP32 inputs."""

import ctypes

import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _outs(R, C, transpose):
    q = torch.full((R, C), 0xAB, dtype=torch.uint8, device=DEV)
    qt = torch.full((C, R), 0xCD, dtype=torch.uint8, device=DEV) if transpose else None
    s = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    return q, qt, s


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_the_workspace_entry_point(dtype):
    lib = fq.lib()
    amax_ref = torch.ones(1, dtype=torch.float32, device=DEV)
    amax_new = torch.ones(1, dtype=torch.float32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xt = fq.IN_BF16 if dtype == torch.bfloat16 else fq.IN_F32
    # the second call is smaller: fewer partial maxima than the first call left in the scratch
    for step, (R, C, transpose, mag) in enumerate([(4096, 2048, True, 3.0), (384, 256, False, 0.02)]):
        x = (synth.random_f32((R, C), seed=60 + step, std=mag) if dtype == torch.float32
             else synth.random_bf16((R, C), seed=60 + step, std=mag)).to(DEV)
        q_ref, qt_ref, s_ref = _outs(R, C, transpose)
        q_new, qt_new, s_new = _outs(R, C, transpose)
        ws = torch.empty(fq.fp8bq_quantize_tensor_workspace_size(R, C), dtype=torch.uint8, device=DEV)
        st = lib.fp8bq_quantize_tensor_delayed(_ptr(x), xt, R, C, C, fq.E4M3, _ptr(amax_ref), 0.99, _ptr(q_ref), C,
                                               _ptr(qt_ref), R if transpose else 0, _ptr(s_ref), _ptr(ws),
                                               ws.numel(), stream)
        assert st == 0, fq.status_string(st)
        st = lib.fp8bq_quantize_tensor_delayed_noalloc(_ptr(x), xt, R, C, C, fq.E4M3, _ptr(amax_new), 0.99,
                                                       _ptr(q_new), C, _ptr(qt_new), R if transpose else 0,
                                                       _ptr(s_new), stream)
        assert st == 0, fq.status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(amax_new.view(torch.int32), amax_ref.view(torch.int32)), f"step {step}: running amax"
        assert torch.equal(s_new.view(torch.int32), s_ref.view(torch.int32)), f"step {step}: scale"
        assert torch.equal(q_new, q_ref), f"step {step}: codes"
        if transpose:
            assert torch.equal(qt_new, qt_ref), f"step {step}: transposed codes"


def test_noalloc_validates_like_the_workspace_entry_point():
    lib = fq.lib()
    x = torch.zeros((128, 128), dtype=torch.bfloat16, device=DEV)
    q, qt, s = _outs(128, 128, True)
    amax = torch.ones(1, dtype=torch.float32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lambda **kw: lib.fp8bq_quantize_tensor_delayed_noalloc(
        kw.get("x", _ptr(x)), 0, 128, kw.get("C", 128), 128, 0, _ptr(amax), kw.get("beta", 0.5), _ptr(q), 128,
        _ptr(qt), 128, kw.get("s", _ptr(s)), stream)
    assert call(C=100) == 2                       # FP8BQ_ERR_SHAPE
    assert call(beta=1.5) == 11                   # FP8BQ_ERR_VALUE
    assert call(x=ctypes.c_void_p(0)) == 1        # FP8BQ_ERR_NULL
    assert call(s=_ptr(q)) == 10                  # FP8BQ_ERR_OVERLAP: the scale inside the codes
    torch.cuda.synchronize()
    assert torch.all(q == 0xAB) and float(amax.item()) == 1.0  # nothing ran
