"""Per-tensor delayed scaling: a running (EMA) amax and one FP8 scale per
tensor, and the GEMM of two per-tensor-scaled operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: [HL] section "核心挑战：Scale Factor 管理", the ``FP8Linear``
listing, which keeps one running amax per tensor in a one-element fp32
buffer:

* amax update (``_update_amax``): the buffer is decayed by beta and the
  tensor's current max |x| is added with weight (1 - beta).  In the listing
  these are two in-place torch operations on the fp32 buffer, so each
  product and the sum round to fp32 separately (no fused multiply-add), and
  beta and 1 - beta enter as fp32 constants (1 - beta is formed in Python
  double first).  The listing's default beta is 0.99 and its buffers start
  at 1.0.
* the type of the weighted current amax: the listing takes max |x| of the
  tensor as given and multiplies it by (1 - beta) before adding it to the
  buffer, so that product has the tensor's own type.  For an FP32 tensor it
  is fp32(cur * (1 - beta)); for a BF16 tensor torch forms the product in
  fp32 and rounds it to BF16 (ties to even), and the fp32 buffer then adds
  that BF16 value.  The oracle follows the listing literally: callers state
  the tensor's type (``in_dtype`` "bf16" or "f32").
* order (``forward``): both running amaxes are updated first, and each
  tensor is then quantized with its updated amax.  The current amax is taken
  from the tensor as given, while the quantized values are those of its
  BF16 copy (the listing quantizes ``x.bfloat16()`` and
  ``weight.bfloat16()``).
* scale and codes (``_quantize``): s = max(fp32(amax / fmt_max),
  fp32(1e-12)); q = nearest FP8 code (ties to even) of
  clamp(fp32(bf16(x) / s), +-fmt_max).  The listing names only E4M3
  (fmt_max 448); E5M2 uses 57344, as for the blockwise rule.
* product: the listing dequantizes (code times scale) and contracts; its
  production note (section "实际生产建议") runs the contraction as an FP8
  GEMM with the two per-tensor scales.  Here that GEMM is the exact float64
  product of the dequantized operands.

Inputs are NumPy arrays holding fp32 (or BF16-valued fp32) numbers.
"""

import numpy as np

from .fp8_codec import decode, encode, fmt_max
from .gemm import to_bf16_rne
from .quant import SCALE_FLOOR


def ema_constants(beta):
    """The fp32 multipliers (beta, 1 - beta) of the running-amax update; 1 - beta is formed
    in double precision before it is rounded to fp32."""
    return np.float32(beta), np.float32(1.0 - float(beta))


IN_DTYPES = ("bf16", "f32")


def amax_ema_update(amax, x, beta, in_dtype):
    """New running amax after seeing tensor x (its values as fp32 numbers; in_dtype is the type
    the tensor has, "bf16" or "f32"):
        fresh = fp32(max|x| * (1 - beta)), rounded to BF16 when the tensor is BF16;
        amax' = fp32(fp32(amax * beta) + fresh)."""
    if in_dtype not in IN_DTYPES:
        raise ValueError(f"in_dtype must be one of {IN_DTYPES}")
    x = np.asarray(x, dtype=np.float32)
    if x.size == 0:
        raise ValueError("the running amax is not updated by an empty tensor")
    cur = np.float32(np.max(np.abs(x)))
    b1, b2 = ema_constants(beta)
    decayed = np.float32(np.float32(amax) * b1)
    fresh = np.float32(cur * b2)
    if in_dtype == "bf16":
        fresh = np.float32(to_bf16_rne(np.array([fresh], np.float32))[0])
    return np.float32(decayed + fresh)


def tensor_scale(amax, fmt):
    """Per-tensor scale from a running amax: max(fp32(amax / fmt_max), fp32(1e-12))."""
    s = np.float32(np.float32(amax) / np.float32(fmt_max(fmt)))
    return np.float32(max(s, SCALE_FLOOR))


def quant_tensor(x, s, fmt):
    """Codes of the BF16 copy of x under the per-tensor scale s (x any shape)."""
    xb = to_bf16_rne(np.asarray(x, dtype=np.float32)).astype(np.float32)  # exact: BF16 values fit fp32
    fmax = np.float32(fmt_max(fmt))
    y = (xb / np.float32(s)).astype(np.float32)  # IEEE fp32 divide
    y = np.minimum(np.maximum(y, -fmax), fmax).astype(np.float32)
    return encode(y, fmt)


def quant_tensor_delayed(x, amax, beta, fmt, in_dtype):
    """One step of the listing for one tensor of type in_dtype ("bf16" or "f32"): update the
    running amax with x, then quantize x.

    Returns (codes uint8 like x, scale float32, new running amax float32).
    """
    a = amax_ema_update(amax, x, beta, in_dtype)
    s = tensor_scale(a, fmt)
    return quant_tensor(x, s, fmt), s, a


def dequant_tensor(q, s, fmt):
    """float64 values decode(q) * s."""
    return decode(np.asarray(q, dtype=np.uint8), fmt) * np.float64(np.float32(s))


def gemm_tensor(qa, sa, fa, qb, sb, fb):
    """Y64[m, n] = sa * sb * sum_k dec(qa[m, k]) dec(qb[n, k]), unrounded float64 (both operands
    contiguous along the contraction, as Y = A . B^T)."""
    return dequant_tensor(qa, sa, fa) @ dequant_tensor(qb, sb, fb).T
