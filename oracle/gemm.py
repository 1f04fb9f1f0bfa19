"""FP8 blockwise GEMMs (fprop, dgrad, wgrad) as float64 contractions of the
dequantized operands, and exact BF16 rounding of the result.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the method computes: the linear layer's three products on FP8 operands
with per-block FP32 scales, accumulated in high precision and written out in
BF16 ([XZY] paragraph "FP8发挥RTX 5090的低精度效率优势"; [APD] "方法关键点",
bullet "FP8 blockwise 混合精度").  [HL] ``FP8Linear.forward`` defines the
product as dequantize-then-contract: both operands are decoded, multiplied
by their scales, and fed to an ordinary matmul.  That is the plain
definition written out here, in float64:

    A_dq = decode(qA) * s_A   (each scale broadcast over its block)
    Y64  = A_dq @ B_dq^T      (NumPy float64 matmul)
    Y    = bf16_rne(Y64)

Summing per 128-wide contraction block, Y = sum_kb s_A s_B sum_{k in kb}
dec(qA) dec(qB), is the same number up to float64 rounding; the
``*_blockloops`` functions evaluate that form literally and the tests check
the two agree.

Shapes (W is [out, in] as in the listing's ``F.linear``):

* fprop:  Y[M, N]  = X[M, K]  . W[N, K]^T   X in 1x128 groups, W in 128x128
* dgrad:  dX[M, K] = dY[M, N] . W[N, K]     dY in 1x128 groups (along N)
* wgrad:  dW[N, K] = dY[M, N]^T . X[M, K]   dY and X in 128x1 groups (along M)
"""

import numpy as np

from .fp8_codec import decode

GROUP = 128


# ---------------------------------------------------------------------------
# BF16 rounding (output precision).  Round-to-nearest-even directly from
# float64 (never through fp32, which would round twice).
# ---------------------------------------------------------------------------

def to_bf16_rne(v):
    """float64 values of the nearest BF16 numbers (ties to even)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)  # v = m * 2**e, 0.5 <= |m| < 1
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # 8 significant bits
    sub = np.ldexp(np.rint(np.ldexp(v, 133)), -133)  # fixed quantum 2**-133
    out = np.where(e >= -125, normal, sub)
    if np.any(np.abs(out) > 3.3895313892515355e38):
        raise OverflowError("value beyond the BF16 range")
    return out


def bf16_bits_to_f64(bits):
    """float64 values of raw BF16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Dequantization: decode(q) * s with each scale broadcast over its block.
# ---------------------------------------------------------------------------

def dequant_act_1x128(q, s, fmt):
    """q[R, C], s[R, C/128] -> float64[R, C]."""
    q = np.asarray(q, np.uint8)
    s = np.asarray(s, np.float32).astype(np.float64)
    return decode(q, fmt) * np.repeat(s, GROUP, axis=1)


def dequant_act_128x1(q, s, fmt):
    """q[R, C] (x's orientation), s[R/128, C] -> float64[R, C]."""
    q = np.asarray(q, np.uint8)
    s = np.asarray(s, np.float32).astype(np.float64)
    return decode(q, fmt) * np.repeat(s, GROUP, axis=0)


def dequant_weight_128x128(q, s, fmt):
    """q[N, K], s[N/128, K/128] -> float64[N, K]."""
    q = np.asarray(q, np.uint8)
    s = np.asarray(s, np.float32).astype(np.float64)
    return decode(q, fmt) * np.repeat(np.repeat(s, GROUP, axis=0), GROUP, axis=1)


# ---------------------------------------------------------------------------
# GEMMs: float64 contraction of the dequantized operands.
# ---------------------------------------------------------------------------

def gemm_fprop(qx, sx, fx, qw, sw, fw):
    """Y64[M, N] = X_dq . W_dq^T  (unrounded float64)."""
    return dequant_act_1x128(qx, sx, fx) @ dequant_weight_128x128(qw, sw, fw).T


def gemm_dgrad(qdy, sdy, fdy, qw, sw, fw):
    """dX64[M, K] = dY_dq . W_dq  (dY in 1x128 groups along N)."""
    return dequant_act_1x128(qdy, sdy, fdy) @ dequant_weight_128x128(qw, sw, fw)


def gemm_wgrad(qdy, sdy, fdy, qx, sx, fx):
    """dW64[N, K] = dY_dq^T . X_dq  (both in 128x1 groups along M).

    qdy[M, N], qx[M, K] are in the original orientation; sdy[M/128, N],
    sx[M/128, K].
    """
    return dequant_act_128x1(qdy, sdy, fdy).T @ dequant_act_128x1(qx, sx, fx)


# ---------------------------------------------------------------------------
# The same products summed block by block, scales applied per block.
# ---------------------------------------------------------------------------

def gemm_fprop_blockloops(qx, sx, fx, qw, sw, fw):
    """Y[m, n] = sum_kb sx[m, kb] sw[n/128, kb] sum_{k in kb} dx[m, k] dw[n, k]."""
    dx, dw = decode(qx, fx), decode(qw, fw)
    M, K = dx.shape
    N = dw.shape[0]
    sx = np.asarray(sx, np.float32).astype(np.float64)
    sw = np.asarray(sw, np.float32).astype(np.float64)
    y = np.zeros((M, N))
    for kb in range(K // GROUP):
        ks = slice(kb * GROUP, (kb + 1) * GROUP)
        t = dx[:, ks] @ dw[:, ks].T
        scale = sx[:, kb][:, None] * np.repeat(sw[:, kb], GROUP)[None, :]
        y += scale * t
    return y


def gemm_dgrad_blockloops(qdy, sdy, fdy, qw, sw, fw):
    """dX[m, k] = sum_nb sdy[m, nb] sw[nb, k/128] sum_{n in nb} ddy[m, n] dw[n, k]."""
    ddy, dw = decode(qdy, fdy), decode(qw, fw)
    M, N = ddy.shape
    K = dw.shape[1]
    sdy = np.asarray(sdy, np.float32).astype(np.float64)
    sw = np.asarray(sw, np.float32).astype(np.float64)
    y = np.zeros((M, K))
    for nb in range(N // GROUP):
        ns = slice(nb * GROUP, (nb + 1) * GROUP)
        t = ddy[:, ns] @ dw[ns, :]
        scale = sdy[:, nb][:, None] * np.repeat(sw[nb, :], GROUP)[None, :]
        y += scale * t
    return y


def gemm_wgrad_blockloops(qdy, sdy, fdy, qx, sx, fx):
    """dW[n, k] = sum_mb sdy[mb, n] sx[mb, k] sum_{m in mb} ddy[m, n] dx[m, k]."""
    ddy, dx = decode(qdy, fdy), decode(qx, fx)
    M, N = ddy.shape
    K = dx.shape[1]
    sdy = np.asarray(sdy, np.float32).astype(np.float64)
    sx = np.asarray(sx, np.float32).astype(np.float64)
    y = np.zeros((N, K))
    for mb in range(M // GROUP):
        ms = slice(mb * GROUP, (mb + 1) * GROUP)
        t = ddy[ms, :].T @ dx[ms, :]
        y += (sdy[mb, :][:, None] * sx[mb, :][None, :]) * t
    return y
