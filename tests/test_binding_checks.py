"""The Python binding refuses, before any launch, tensors that the C ABI cannot check itself (the C
calls see only pointers and leading dimensions): a wrong element type, a shape other than the one
the call implies (an output with too few rows, a scale array of the wrong orientation, an FP32
main-grad buffer that is BF16), or a tensor on another device.  Runs on the CPU: the checks come
before the library is called, and the outputs are left as they were."""

import pytest
import torch

import fp8_blockwise_quantized_amd as fq

M, N, K = 256, 384, 512


def _u8(*shape):
    return torch.full(shape, 7, dtype=torch.uint8)


def _f32(*shape):
    return torch.full(shape, 0.5, dtype=torch.float32)


def _bf16(*shape):
    return torch.full(shape, 2.0, dtype=torch.bfloat16)


def _fprop_args(**over):
    a = dict(qx=_u8(M, K), sx=_f32(K // 128, M), fx=fq.E4M3, qw=_u8(N, K), sw=_f32(N // 128, K // 128), fw=fq.E4M3,
             y=_bf16(M, N))
    a.update(over)
    return a


@pytest.mark.parametrize("bad,exc", [
    (dict(y=_bf16(M - 1, N)), ValueError),               # too few output rows
    (dict(y=torch.zeros((M, N), dtype=torch.float16)), TypeError),
    (dict(sx=_f32(M, K // 128)), ValueError),             # scales in the wrong orientation
    (dict(sx=torch.zeros((K // 128, M), dtype=torch.bfloat16)), TypeError),
    (dict(qw=_u8(N, K - 128)), ValueError),
    (dict(qx=torch.zeros((M, K), dtype=torch.int8)), TypeError),
])
def test_gemm_fprop_refuses_mismatched_tensors(bad, exc):
    a = _fprop_args(**bad)
    before = a["y"].clone()
    with pytest.raises(exc):
        fq.fp8bq_gemm_fprop(a["qx"], a["sx"], a["fx"], a["qw"], a["sw"], a["fw"], a["y"])
    assert torch.equal(a["y"], before)


def test_host_tensors_are_refused():
    a = _fprop_args()
    with pytest.raises(ValueError, match="CUDA"):
        fq.fp8bq_gemm_fprop(a["qx"], a["sx"], a["fx"], a["qw"], a["sw"], a["fw"], a["y"])


def test_wgrad_accumulate_needs_an_fp32_buffer_of_the_output_shape():
    qdyt, sdyt, qxt, sxt = _u8(N, M), _f32(M // 128, N), _u8(K, M), _f32(M // 128, K)
    with pytest.raises(TypeError):
        fq.fp8bq_gemm_wgrad(qdyt, sdyt, fq.E4M3, qxt, sxt, fq.E4M3, _bf16(N, K), accumulate=True)
    with pytest.raises(ValueError):
        fq.fp8bq_gemm_wgrad(qdyt, sdyt, fq.E4M3, qxt, sxt, fq.E4M3, _f32(N, K - 128), accumulate=True)


@pytest.mark.parametrize("call", [
    lambda: fq.fp8bq_quantize_act_1x128(_bf16(M, K), fq.E4M3, _u8(M, K), _f32(M, K // 128)),
    lambda: fq.fp8bq_quantize_act_128x1(_bf16(M, K), fq.E4M3, _u8(M, K), _f32(M // 128, K)),
    lambda: fq.fp8bq_quantize_act_dual(_bf16(M, K), fq.E4M3, _u8(M, K), _f32(K // 128, M), fq.E4M3, _u8(K, M),
                                       _f32(K // 128, M)),
    lambda: fq.fp8bq_quantize_weight_dual(_bf16(N, K), fq.E4M3, _u8(N, K), _f32(N // 128, K // 128), _u8(N, K)),
    lambda: fq.fp8bq_quantize_weight_128x128(_bf16(N, K), fq.E4M3, _u8(N, K), _f32(K // 128, N // 128)),
    lambda: fq.fp8bq_gemm_dgrad(_u8(M, N), _f32(N // 128, M), fq.E4M3, _u8(N, K), _f32(N // 128, K // 128), fq.E4M3,
                                _bf16(M, N)),
    lambda: fq.fp8bq_gemm_dgrad_wt(_u8(M, N), _f32(N // 128, M), fq.E4M3, _u8(N, K), _f32(N // 128, K // 128),
                                   fq.E4M3, _bf16(M, K)),
    lambda: fq.fp8bq_quantize_tensor_delayed(_bf16(M, K), fq.E4M3, _f32(2), 0.99, _u8(M, K), None, _f32(1), _u8(64)),
    lambda: fq.fp8bq_quantize_tensor_delayed_noalloc(_bf16(M, K), fq.E4M3, _f32(1), 0.99, _u8(M, K), _u8(M, K),
                                                     _f32(1)),
    lambda: fq.fp8bq_gemm_tensor(_u8(M, K), _f32(1), fq.E4M3, _u8(N, K), _f32(1), fq.E4M3, _bf16(N, M)),
    lambda: fq.fp8bq_hyperball_step(_f32(N, K), _bf16(N, K), 1e-4, 0.1, 1e-8, 0.0, _f32(3), _u8(64)),
    lambda: fq.fp8bq_hyperball_step(_bf16(N, K), _bf16(N, K), 1e-4, 0.1, 1e-8, 0.0, None, _u8(64)),
])
def test_every_entry_point_checks_its_tensors(call):
    with pytest.raises((TypeError, ValueError)) as e:
        call()
    assert "CUDA" not in str(e.value)  # refused for its dtype or shape, before the device check


def test_prepare_validates_once_up_front():
    a = _fprop_args(y=_bf16(M - 1, N))
    with pytest.raises(ValueError):
        fq.prepare(fq.fp8bq_gemm_fprop, a["qx"], a["sx"], a["fx"], a["qw"], a["sw"], a["fw"], a["y"])
