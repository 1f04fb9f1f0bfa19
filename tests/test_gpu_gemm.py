"""GPU parity of the scaled FP8 GEMMs (fprop, dgrad, wgrad) against the float64 oracle.

Every case quantizes on the GPU and in the oracle from the same seeded inputs (the codes are
bit-identical, checked separately), runs the GPU GEMM, and holds each sampled output to
|err| <= 2e-3 ||a_i|| ||b_j|| and a relative Frobenius error <= 1e-3 against the BF16-rounded
float64 result (FP32 outputs to 1e-4 of the same bound; degenerate parallel-row inputs to the bound
on the error beyond the BF16 output rounding).  Small cases compare every output; the
full-size workloads compare sampled rows / columns computed one by one by the oracle.
"""

import os

import numpy as np
import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import oracle
import synth
from parity import FP, check_gemm, row_norms, say, to_np_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TILE_FORCED = "FP8BQ_GEMM_TILE" in os.environ  # the planner's tile choice is overridden (tuning runs)
E4, E5 = oracle.E4M3, oracle.E5M2


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)]))
    return idx


# ------------------------------------------------------------------------------------------
# end-to-end helpers: GPU quantize + GEMM, oracle quantize + GEMM on the sampled slice
# ------------------------------------------------------------------------------------------

def run_fprop(X, W, fx=E4, fw=E4, rows=None, out_dtype=torch.bfloat16):
    Xd, Wd = X.to(DEV), W.to(DEV)
    qx, sx = fq.quantize_act_1x128(Xd, FP[fx])
    qw, sw = fq.quantize_weight_128x128(Wd, FP[fw])
    y = fq.gemm_fprop(qx, sx, qw, sw, FP[fx], FP[fw], out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = np.arange(X.shape[0]) if rows is None else rows
    oqx, osx = oracle.quant_act_1x128(X[rows].float().numpy(), fx)
    oqw, osw = oracle.quant_weight_128x128(W.float().numpy(), fw)
    a = oracle.dequant_act_1x128(oqx, osx, fx)
    b = oracle.dequant_weight_128x128(oqw, osw, fw)
    y64 = a @ b.T
    return to_np_f64(y[torch.from_numpy(rows).to(DEV)]), y64, row_norms(a), row_norms(b)


def run_dgrad(dY, W, fdy=E4, fw=E4, rows=None, out_dtype=torch.bfloat16):
    dYd, Wd = dY.to(DEV), W.to(DEV)
    qdy, sdy = fq.quantize_act_1x128(dYd, FP[fdy])
    qw, sw = fq.quantize_weight_128x128(Wd, FP[fw])
    dx = fq.gemm_dgrad(qdy, sdy, qw, sw, FP[fdy], FP[fw], out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = np.arange(dY.shape[0]) if rows is None else rows
    oq, os_ = oracle.quant_act_1x128(dY[rows].float().numpy(), fdy)
    oqw, osw = oracle.quant_weight_128x128(W.float().numpy(), fw)
    a = oracle.dequant_act_1x128(oq, os_, fdy)
    b = oracle.dequant_weight_128x128(oqw, osw, fw)
    y64 = a @ b
    return to_np_f64(dx[torch.from_numpy(rows).to(DEV)]), y64, row_norms(a), row_norms(b.T)


def run_wgrad(dY, X, fdy=E4, fx=E4, ncols=None, kcols=None, out_dtype=torch.bfloat16):
    dYd, Xd = dY.to(DEV), X.to(DEV)
    qdyt, sdyt = fq.quantize_act_128x1(dYd, FP[fdy])
    qxt, sxt = fq.quantize_act_128x1(Xd, FP[fx])
    dw = fq.gemm_wgrad(qdyt, sdyt, qxt, sxt, FP[fdy], FP[fx], out_dtype=out_dtype)
    torch.cuda.synchronize()
    ncols = np.arange(dY.shape[1]) if ncols is None else ncols
    kcols = np.arange(X.shape[1]) if kcols is None else kcols
    oq, os_ = oracle.quant_act_128x1(np.ascontiguousarray(dY[:, ncols].float().numpy()), fdy)
    oqx, osx = oracle.quant_act_128x1(np.ascontiguousarray(X[:, kcols].float().numpy()), fx)
    a = oracle.dequant_act_128x1(oq, os_, fdy)   # [M, n]
    b = oracle.dequant_act_128x1(oqx, osx, fx)   # [M, k]
    y64 = a.T @ b
    got = to_np_f64(dw)[np.ix_(ncols, kcols)]
    return got, y64, row_norms(a.T), row_norms(b.T)


def checked(res, what, out_f32=False):
    got, y64, an, bn = res
    worst, fro = check_gemm(got, y64, an, bn, out_f32=out_f32, what=what)
    say(f"{what}: max|err|/(|a||b|) = {worst:.2e}, rel Frobenius = {fro:.2e}")


# ------------------------------------------------------------------------------------------
# tiny workload: every output compared
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_tiny_workload_all_products(out_dtype):
    c = synth.tiny_check()
    f32 = out_dtype == torch.float32
    checked(run_fprop(c["A"], c["W"], out_dtype=out_dtype), "tiny fprop", f32)
    checked(run_dgrad(c["dY"], c["W"], E5, E4, out_dtype=out_dtype), "tiny dgrad e5m2", f32)
    checked(run_dgrad(c["dY"], c["W"], E4, E4, out_dtype=out_dtype), "tiny dgrad e4m3", f32)
    checked(run_wgrad(c["dY"], c["A"], E4, E4, out_dtype=out_dtype), "tiny wgrad", f32)
    checked(run_wgrad(c["dY"], c["A"], E5, E4, out_dtype=out_dtype), "tiny wgrad e5m2", f32)


def test_gemm_on_oracle_codes():
    """The GEMM alone: the oracle's codes and scales are uploaded, so no GPU quantizer is involved."""
    c = synth.tiny_check()
    qx, sx = oracle.quant_act_1x128(c["A"].numpy(), E4)
    qw, sw = oracle.quant_weight_128x128(c["W"].numpy(), E4)
    tq = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    y = fq.gemm_fprop(tq(qx), tq(sx.T), tq(qw), tq(sw))
    torch.cuda.synchronize()
    a = oracle.dequant_act_1x128(qx, sx, E4)
    b = oracle.dequant_weight_128x128(qw, sw, E4)
    checked((to_np_f64(y), a @ b.T, row_norms(a), row_norms(b)), "fprop on oracle codes")


def test_bf16_output_is_rne_of_fp32_accumulator():
    X = synth.random_bf16((300, 512), seed=41, outliers=True)
    W = synth.random_bf16((384, 512), seed=42, std=0.02)
    Xd, Wd = X.to(DEV), W.to(DEV)
    qx, sx = fq.quantize_act_1x128(Xd)
    qw, sw = fq.quantize_weight_128x128(Wd)
    y16 = fq.gemm_fprop(qx, sx, qw, sw, out_dtype=torch.bfloat16)
    y32 = fq.gemm_fprop(qx, sx, qw, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    exp = oracle.to_bf16_rne(y32.cpu().numpy().astype(np.float64))
    assert np.array_equal(to_np_f64(y16), exp)


# ------------------------------------------------------------------------------------------
# ragged, multi-tile and strided shapes
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 17, 100, 129, 300, 1000])
def test_fprop_ragged_tokens(M):
    X = synth.random_bf16((M, 384), seed=M, outliers=True)
    W = synth.random_bf16((640, 384), seed=M + 1, std=0.02)
    checked(run_fprop(X, W), f"fprop M={M}")


@pytest.mark.parametrize("M", [1, 33, 130, 515])
@pytest.mark.parametrize("fdy", [E4, E5])
def test_dgrad_ragged_tokens(M, fdy):
    dY = synth.random_bf16((M, 512), seed=M + 7, std=1e-3)
    W = synth.random_bf16((512, 384), seed=M + 8, std=0.02)
    checked(run_dgrad(dY, W, fdy, E4), f"dgrad M={M} {fdy}")


@pytest.mark.parametrize("shape", [(128, 128, 128), (256, 384, 256), (512, 128, 640), (1024, 256, 384)])
@pytest.mark.parametrize("fdy", [E4, E5])
def test_wgrad_shapes(shape, fdy):
    M, N, K = shape
    dY = synth.random_bf16((M, N), seed=1000 + M + N, std=1e-3)
    X = synth.random_bf16((M, K), seed=2000 + M + K, outliers=True)
    checked(run_wgrad(dY, X, fdy, E4), f"wgrad {shape} {fdy}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_wgrad_parallel_rows(out_dtype):
    """dY and X drawn from one stream, so column c of dY is parallel to column c of X and the
    diagonal of dW equals ||a|| ||b||: every product in those sums has the same sign.  Held to the
    bound on the error beyond the output rounding (BF16 rounding alone reaches 2^-8 relative)."""
    dY = synth.random_bf16((256, 128), seed=5, std=1e-3)
    X = synth.random_bf16((256, 128), seed=5)
    got, y64, an, bn = run_wgrad(dY, X, E4, E4, out_dtype=out_dtype)
    f32 = out_dtype == torch.float32
    worst, _ = check_gemm(got, y64, an, bn, out_f32=f32, what="parallel rows", beyond_rounding=not f32)
    say(f"parallel rows {out_dtype}: max |err| / (|a||b|) = {worst:.2e}")


@pytest.mark.parametrize("fx,fw", [(E5, E5), (E4, E5)])
def test_fprop_other_format_pairs(fx, fw):
    X = synth.random_bf16((200, 256), seed=51, outliers=True)
    W = synth.random_bf16((256, 256), seed=52, std=0.02)
    checked(run_fprop(X, W, fx, fw), f"fprop {fx}x{fw}")


def test_strided_operands_and_output():
    X = synth.random_bf16((300, 256), seed=61, outliers=True).to(DEV)
    W = synth.random_bf16((256, 256), seed=62, std=0.02).to(DEV)
    qx, sx = fq.quantize_act_1x128(X)
    qw, sw = fq.quantize_weight_128x128(W)
    qx_big = torch.zeros((300, 384), dtype=torch.uint8, device=DEV)
    qx_big[:, :256] = qx
    y_big = torch.full((300, 272), -7.0, dtype=torch.bfloat16, device=DEV)
    y = y_big[:, :256]
    fq.fp8bq_gemm_fprop(qx_big[:, :256], sx, fq.E4M3, qw, sw, fq.E4M3, y)
    ref = fq.gemm_fprop(qx, sx, qw, sw)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    assert torch.all(y_big[:, 256:] == -7.0)  # padding untouched


def test_empty_and_zero_contraction():
    y = torch.full((64, 128), 5.0, dtype=torch.bfloat16, device=DEV)
    qx = torch.empty((64, 0), dtype=torch.uint8, device=DEV)
    sx = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    qw = torch.empty((128, 0), dtype=torch.uint8, device=DEV)
    sw = torch.empty((1, 0), dtype=torch.float32, device=DEV)
    lib = fq.lib()
    st = lib.fp8bq_gemm_fprop(64, 128, 0, None, 16, None, 64, 0, None, 16, None, 1, 0, y.data_ptr(), 0, 128, None,
                              0, None)
    torch.cuda.synchronize()
    assert st == 0 and torch.all(y == 0)
    # no rows: nothing written, nothing read
    st = lib.fp8bq_gemm_fprop(0, 128, 256, None, 256, None, 4, 0, None, 256, None, 2, 0, None, 0, 128, None, 0, None)
    assert st == 0
    del qx, sx, qw, sw


def test_deterministic():
    X = synth.random_bf16((512, 1024), seed=71).to(DEV)
    W = synth.random_bf16((512, 1024), seed=72, std=0.02).to(DEV)
    qx, sx = fq.quantize_act_1x128(X)
    qw, sw = fq.quantize_weight_128x128(W)
    a = fq.gemm_fprop(qx, sx, qw, sw)
    b = fq.gemm_fprop(qx, sx, qw, sw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------------------------------
# full-size workloads, sampled outputs
# ------------------------------------------------------------------------------------------

def test_single_linear_fprop_full_size():
    c = synth.single_linear()
    rows = _sample(8192, 192, 1)
    checked(run_fprop(c["X"], c["W"], rows=rows), "8192x8192x2048 fprop (sampled rows)")


@pytest.mark.parametrize("name", [n for n, _, _ in synth.DECODER_LINEARS])
def test_decoder_block_full_size(name):
    say(f"decoder block linear {name}")
    c = synth.decoder_linear(name)
    M, K = c["X"].shape
    N = c["W"].shape[0]
    rows = _sample(M, 96, 2)
    checked(run_fprop(c["X"], c["W"], rows=rows), f"{name} fprop")
    checked(run_dgrad(c["dY"], c["W"], rows=rows), f"{name} dgrad")
    checked(run_wgrad(c["dY"], c["X"], ncols=_sample(N, 48, 3), kcols=_sample(K, 48, 4)), f"{name} wgrad")


def test_sweep_fprop_all_sizes():
    W = synth.sweep_weight()
    for M in synth.SWEEP_M:
        X = synth.sweep_x(M)
        checked(run_fprop(X, W, rows=_sample(M, 64, M)), f"sweep fprop M={M}")


def test_heavy_tailed_gradients_full_size():
    c = synth.heavy_tailed()
    rows = _sample(16384, 96, 5)
    checked(run_dgrad(c["dY"], c["W"], E5, E4, rows=rows), "heavy-tail dgrad e5m2 x e4m3")
    ncols, kcols = _sample(5632, 48, 6), _sample(2048, 48, 7)
    checked(run_wgrad(c["dY"], c["X"], E5, E4, ncols=ncols, kcols=kcols), "heavy-tail wgrad e5m2 x e4m3")
    checked(run_wgrad(c["dY"], c["X"], E4, E4, ncols=ncols, kcols=kcols), "heavy-tail wgrad e4m3 x e4m3")


@pytest.mark.parametrize("shape", [(256, 256, 2560), (200, 256, 3328), (128, 128, 4096)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_split_contraction(shape, out_dtype):
    """Few output tiles and a long contraction: the planner splits the contraction across work
    units (uneven splits included) and adds the FP32 partial sums in a fixed order."""
    M, N, K = shape
    X = synth.random_bf16((M, K), seed=81 + K, outliers=True)
    W = synth.random_bf16((N, K), seed=82 + K, std=0.02)
    split = fq.fp8bq_gemm_workspace_size(fq.OP_FPROP, M, N, K)
    assert split > 0  # this shape takes the split path
    checked(run_fprop(X, W, out_dtype=out_dtype), f"split fprop {shape}", out_dtype == torch.float32)
    if M % 128 == 0:  # wgrad's output dimensions are feature counts (multiples of 128)
        dY = synth.random_bf16((K, N), seed=83 + K, std=1e-3)
        Xw = synth.random_bf16((K, M), seed=84 + K, outliers=True)
        checked(run_wgrad(dY, Xw, out_dtype=out_dtype), f"split wgrad {shape}", out_dtype == torch.float32)
    dYd = synth.random_bf16((M, K), seed=85 + K, std=1e-3)
    Wd = synth.random_bf16((K, N), seed=86 + K, std=0.02)
    checked(run_dgrad(dYd, Wd, out_dtype=out_dtype), f"split dgrad {shape}", out_dtype == torch.float32)


def test_split_is_deterministic():
    dY = synth.random_bf16((4096, 256), seed=91, std=1e-3).to(DEV)
    X = synth.random_bf16((4096, 256), seed=92).to(DEV)
    qdyt, sdyt = fq.quantize_act_128x1(dY)
    qxt, sxt = fq.quantize_act_128x1(X)
    a = fq.gemm_wgrad(qdyt, sdyt, qxt, sxt)
    b = fq.gemm_wgrad(qdyt, sdyt, qxt, sxt)
    torch.cuda.synchronize()
    assert fq.fp8bq_gemm_workspace_size(fq.OP_WGRAD, 4096, 256, 256) > 0
    assert torch.equal(a, b)


# ------------------------------------------------------------------------------------------
# the 256x256 tile path with ragged tiles (rows past M, columns past N) and split partials
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_large_tile_ragged_edges(out_dtype):
    """Shapes the planner runs on 256x256 tiles whose last tile row and column reach past the
    output (4200 = 16*256 + 104 rows; 2432 = 9.5 tiles of columns); every output compared."""
    f32 = out_dtype == torch.float32
    M, N, K = 4200, 2432, 2048
    assert TILE_FORCED or fq.fp8bq_gemm_plan(fq.OP_FPROP, M, N, K)[:2] == (256, 256)
    X = synth.random_bf16((M, K), seed=301, outliers=True)
    W = synth.random_bf16((N, K), seed=302, std=0.02)
    checked(run_fprop(X, W, out_dtype=out_dtype), "256x256 ragged fprop", f32)
    Md, Nd, Kd = 4200, 2048, 2432
    assert TILE_FORCED or fq.fp8bq_gemm_plan(fq.OP_DGRAD, Md, Nd, Kd)[:2] == (256, 256)
    dY = synth.random_bf16((Md, Nd), seed=303, std=1e-3)
    Wd = synth.random_bf16((Nd, Kd), seed=304, std=0.02)
    checked(run_dgrad(dY, Wd, out_dtype=out_dtype), "256x256 ragged dgrad", f32)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mid_tile_ragged_edges(out_dtype):
    """Shapes the planner runs on 128x128 tiles whose last tile row reaches past the output
    (1100 = 8*128 + 76 rows); every output compared."""
    f32 = out_dtype == torch.float32
    M, N, K = 1100, 3072, 768
    assert TILE_FORCED or fq.fp8bq_gemm_plan(fq.OP_FPROP, M, N, K) == (128, 128, 1)
    X = synth.random_bf16((M, K), seed=311, outliers=True)
    W = synth.random_bf16((N, K), seed=312, std=0.02)
    checked(run_fprop(X, W, out_dtype=out_dtype), "128x128 ragged fprop", f32)
    assert TILE_FORCED or fq.fp8bq_gemm_plan(fq.OP_DGRAD, M, K, N) == (128, 128, 1)
    dY = synth.random_bf16((M, K), seed=313, std=1e-3)
    Wd = synth.random_bf16((K, N), seed=314, std=0.02)
    checked(run_dgrad(dY, Wd, out_dtype=out_dtype), "128x128 ragged dgrad", f32)


@pytest.mark.parametrize("shape", [(4096, 4480, 2432), (16384, 2944, 1664)])
def test_large_tile_wgrad(shape):
    """wgrad on 256x256 tiles: ragged output columns (2432 = 9.5 tiles) without a split, and ragged
    rows and columns (2944 = 11.5, 1664 = 6.5 tiles) with a split contraction (FP32 partial sums)."""
    M, N, K = shape
    tm, tn, split = fq.fp8bq_gemm_plan(fq.OP_WGRAD, M, N, K)
    assert TILE_FORCED or (tm, tn) == (256, 256)
    assert TILE_FORCED or (split > 1) == (M == 16384)
    dY = synth.random_bf16((M, N), seed=305 + N, std=1e-3)
    X = synth.random_bf16((M, K), seed=306 + K, outliers=True)
    checked(run_wgrad(dY, X, ncols=_sample(N, 160, 7), kcols=_sample(K, 160, 8)), f"256x256 wgrad {shape} split {split}")


# ------------------------------------------------------------------------------------------
# dgrad on pre-transposed weight codes
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(256, 256, 384), (300, 640, 256), (4200, 2048, 2432)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_dgrad_wt_matches_dgrad_and_oracle(shape, out_dtype):
    """fp8bq_gemm_dgrad_wt on the W^T codes of fp8bq_quantize_weight_dual gives fp8bq_gemm_dgrad's
    result bit for bit (same kernel, no transpose pass), and holds the oracle tolerance."""
    M, N, K = shape
    dY = synth.random_bf16((M, N), seed=401 + M, std=1e-3)
    W = synth.random_bf16((N, K), seed=402 + K, std=0.02)
    qdy, sdy = fq.quantize_act_1x128(dY.to(DEV), fq.E5M2)
    qw, sw, qwt = fq.quantize_weight_dual(W.to(DEV), fq.E4M3)
    ref = fq.gemm_dgrad(qdy, sdy, qw, sw, fq.E5M2, fq.E4M3, out_dtype=out_dtype)
    got = fq.gemm_dgrad_wt(qdy, sdy, qwt, sw, fq.E5M2, fq.E4M3, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "dgrad_wt differs from dgrad"
    rows = _sample(M, 128, 9)
    oq, os_ = oracle.quant_act_1x128(dY[rows].float().numpy(), E5)
    oqw, osw = oracle.quant_weight_128x128(W.float().numpy(), E4)
    a = oracle.dequant_act_1x128(oq, os_, E5)
    b = oracle.dequant_weight_128x128(oqw, osw, E4)
    checked((to_np_f64(got[torch.from_numpy(rows).to(DEV)]), a @ b, row_norms(a), row_norms(b.T)),
            f"dgrad_wt {shape}", out_dtype == torch.float32)


# ------------------------------------------------------------------------------------------
# FP32 main-grad accumulation (wgrad epilogue option)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(4096, 256, 256), (512, 2048, 1536), (4096, 4480, 2432)])
def test_wgrad_fp32_accumulate(shape):
    """Two micro-batches accumulated into one FP32 buffer that starts non-zero:
    out = out0 + dW1 + dW2, each GEMM as accurate as the FP32-output wgrad (1e-4 of |a||b|) and each
    addition one FP32 rounding (2^-24 of the running magnitude).  The shapes cover the split
    (partial sums added by the reduction pass) and unsplit (added in the GEMM's own epilogue) paths."""
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    ncols, kcols = np.sort(rng.choice(N, 48, replace=False)), np.sort(rng.choice(K, 48, replace=False))
    out0 = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32) * 0.3)
    out = out0.to(DEV)
    ref = out0.numpy().astype(np.float64)[np.ix_(ncols, kcols)]
    mag = np.abs(ref)
    bound = np.zeros_like(ref)
    for mb in range(2):
        dY = synth.random_bf16((M, N), seed=7000 + 10 * mb + M, std=1e-3)
        X = synth.random_bf16((M, K), seed=7001 + 10 * mb + K, outliers=True)
        qdyt, sdyt = fq.quantize_act_128x1(dY.to(DEV))
        qxt, sxt = fq.quantize_act_128x1(X.to(DEV))
        fq.gemm_wgrad(qdyt, sdyt, qxt, sxt, out=out, accumulate=True)
        oq, os_ = oracle.quant_act_128x1(np.ascontiguousarray(dY[:, ncols].float().numpy()), E4)
        oqx, osx = oracle.quant_act_128x1(np.ascontiguousarray(X[:, kcols].float().numpy()), E4)
        a = oracle.dequant_act_128x1(oq, os_, E4)
        b = oracle.dequant_act_128x1(oqx, osx, E4)
        y64 = a.T @ b
        ref = ref + y64
        mag = mag + np.abs(y64)
        bound = bound + np.outer(row_norms(a.T), row_norms(b.T))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)[np.ix_(ncols, kcols)]
    err = np.abs(got - ref)
    lim = 1e-4 * bound + 2.0 ** -23 * mag
    worst = float(np.max(err / lim))
    assert np.all(err <= lim), f"accumulate {shape}: max err / limit = {worst:.3f}"
    split = fq.fp8bq_gemm_plan(fq.OP_WGRAD, M, N, K)[2]
    say(f"wgrad accumulate {shape} (split {split}): max err / limit = {worst:.3f}")


def test_wgrad_accumulate_paths_and_empty_sum():
    splits = {fq.fp8bq_gemm_plan(fq.OP_WGRAD, *s)[2] > 1 for s in [(4096, 256, 256), (512, 2048, 1536)]}
    assert splits == {True, False}  # the cases above reach both epilogues
    # a zero-length contraction adds nothing: the buffer is left as it was
    out = torch.full((128, 256), 3.25, dtype=torch.float32, device=DEV)
    st = fq.lib().fp8bq_gemm_wgrad(0, 128, 256, None, 16, None, 128, 0, None, 16, None, 256, 0, out.data_ptr(),
                                   fq.OUT_F32_ACCUM, 256, None, 0, None)
    torch.cuda.synchronize()
    assert st == 0 and torch.all(out == 3.25)


# ------------------------------------------------------------------------------------------
# contractions shorter than the LDS ring on 256x256 tiles (1-3 blocks: the ring reloads the last
# block into its free slot; the first unit's prologue already covers the whole contraction)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("K", [128, 256, 384])
def test_short_contraction_on_large_tiles(K):
    M, N = 4096, 4096
    assert TILE_FORCED or fq.fp8bq_gemm_plan(fq.OP_FPROP, M, N, K)[:2] == (256, 256)
    X = synth.random_bf16((M, K), seed=700 + K, outliers=True)
    W = synth.random_bf16((N, K), seed=701 + K, std=0.02)
    checked(run_fprop(X, W, rows=_sample(M, 96, K)), f"fprop K={K} on 256x256 tiles")
    # wgrad over K tokens: dW [4096, 4096] from dY [K, 4096] and X [K, 4096]
    assert TILE_FORCED or fq.fp8bq_gemm_plan(fq.OP_WGRAD, K, N, M)[:2] == (256, 256)
    dY = synth.random_bf16((K, N), seed=702 + K, std=1e-3)
    Xw = synth.random_bf16((K, M), seed=703 + K, outliers=True)
    checked(run_wgrad(dY, Xw, ncols=_sample(N, 96, K + 1), kcols=_sample(M, 96, K + 2)),
            f"wgrad over {K} tokens on 256x256 tiles")


# ------------------------------------------------------------------------------------------
# every operand-format pair through every product, on each kernel form the planner picks
# ------------------------------------------------------------------------------------------

PAIRS = [(E4, E4), (E4, E5), (E5, E4), (E5, E5)]


def _expect_plan(op, shape, plan):
    if not TILE_FORCED:
        assert fq.fp8bq_gemm_plan(op, *shape) == plan, (shape, fq.fp8bq_gemm_plan(op, *shape))


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("shape,plan", [((256, 384, 256), (64, 64, 1)), ((256, 256, 3072), (64, 64, 6)),
                                        ((1024, 4096, 1024), (128, 128, 1)), ((128, 4096, 4096), (128, 128, 4)),
                                        ((4096, 4096, 256), (256, 256, 1))])
def test_fprop_every_format_pair(fa, fb, shape, plan):
    """Each of the four instruction format pairs (the MFMA's per-operand format fields) on every
    kernel form the planner picks: 64x64 and 128x128 tiles, each whole and with a split
    contraction, and 256x256 tiles."""
    M, N, K = shape
    _expect_plan(fq.OP_FPROP, shape, plan)
    X = synth.random_bf16((M, K), seed=3001 + M + K, outliers=True)
    W = synth.random_bf16((N, K), seed=3002 + N + K, std=0.02)
    rows = _sample(M, 192, seed=M) if M > 512 else None
    checked(run_fprop(X, W, fa, fb, rows=rows), f"fprop {shape} {fa}x{fb}")


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("shape,plan", [((256, 384, 256), (64, 64, 1)), ((256, 3072, 256), (64, 64, 6)),
                                        ((1024, 1024, 4096), (128, 128, 1)), ((128, 4096, 4096), (128, 128, 4)),
                                        ((8192, 256, 2048), (256, 256, 1))])
def test_dgrad_every_format_pair(fa, fb, shape, plan):
    M, N, K = shape
    _expect_plan(fq.OP_DGRAD, shape, plan)
    dY = synth.random_bf16((M, N), seed=3003 + M + N, std=1e-3)
    W = synth.random_bf16((N, K), seed=3004 + N + K, std=0.02)
    rows = _sample(M, 192, seed=M + 1) if M > 512 else None
    checked(run_dgrad(dY, W, fa, fb, rows=rows), f"dgrad {shape} {fa}x{fb}")


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("shape,plan", [((256, 384, 256), (64, 64, 1)), ((3072, 256, 256), (64, 64, 6)),
                                        ((1024, 1024, 4096), (128, 128, 1)), ((4096, 128, 4096), (128, 128, 4)),
                                        ((2048, 4096, 4096), (256, 256, 1))])
def test_wgrad_every_format_pair(fa, fb, shape, plan):
    M, N, K = shape
    _expect_plan(fq.OP_WGRAD, shape, plan)
    dY = synth.random_bf16((M, N), seed=3005 + M + N, std=1e-3)
    X = synth.random_bf16((M, K), seed=3006 + M + K, outliers=True)
    ncols = _sample(N, 160, seed=N) if N > 512 else None
    kcols = _sample(K, 160, seed=K + 1) if K > 512 else None
    checked(run_wgrad(dY, X, fa, fb, ncols=ncols, kcols=kcols), f"wgrad {shape} {fa}x{fb}")
