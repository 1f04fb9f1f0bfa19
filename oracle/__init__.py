"""CPU oracle for the FP8 blockwise-quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library under ``fp8_blockwise_quantized_amd/``.

It is deliberately plain and slow: NumPy on the CPU, float64 wherever the
pages do not fix a narrower precision, and no blocking, fusion or reordering
beyond what the definitions state.

Sources (cited by page title and section; the pages are the authority):

* [HL]  "用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析"
        (hankli.space).  Section "Blackwell 的 FP8 Tensor Core" fixes the two
        FP8 formats and their maxima; section "核心挑战：Scale Factor 管理"
        (the ``FP8Linear`` listing, its ``_quantize`` and ``forward``) and
        section "常见错误：直接转换而不加 Scale" fix the quantize rule
        (scale = amax / fmt_max with a 1e-12 floor, divide, clamp, cast) and
        the dequantize rule (code value times scale).
  The same listing's running (EMA) amax with one scale per tensor is the
        per-tensor delayed-scaling variant in ``delayed.py``; its section
        "Hyperball 优化：让 FP8 训练不爆炸" (``HyperballSGD``) is the
        normalized update in ``hyperball.py``.
* [XZY] "小团队也能预训练！普罗2B：RTX5090训练成本不到5090美元" (66bd.net,
        新智元), paragraph "FP8发挥RTX 5090的低精度效率优势": fine-grained
        block quantization after DeepSeek-V3, main linear GEMMs in FP8,
        numerically sensitive state in BF16/FP32.
* [APD] "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090"
        (AI Papers Daily digest), section "方法关键点", bullet
        "FP8 blockwise 混合精度", and section "工作参考价值": E4M3 for the
        transformer linear GEMMs, activations in groups of 128 along one
        axis, weights in 128x128 blocks, sensitive state in BF16/FP32.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
values the pages fix, closed forms, invariants, library routines on special
cases and brute force; none is "parity unpinned" except the heavy-tailed-gradient
quantization-error report, which is reported and not graded.
"""

from .fp8_codec import (  # noqa: F401
    E4M3,
    E5M2,
    FORMATS,
    decode,
    decode_table,
    encode,
    fmt_max,
)
from .quant import (  # noqa: F401
    SCALE_FLOOR,
    quantize_group_rows,
    quant_act_1x128,
    quant_act_128x1,
    quant_weight_128x128,
)
from .gemm import (  # noqa: F401
    to_bf16_rne,
    bf16_bits_to_f64,
    dequant_act_1x128,
    dequant_act_128x1,
    dequant_weight_128x128,
    gemm_fprop,
    gemm_dgrad,
    gemm_wgrad,
    gemm_fprop_blockloops,
    gemm_dgrad_blockloops,
    gemm_wgrad_blockloops,
)
from .delayed import (  # noqa: F401
    amax_ema_update,
    dequant_tensor,
    ema_constants,
    gemm_tensor,
    quant_tensor,
    quant_tensor_delayed,
    tensor_scale,
)
from .hyperball import hyperball_step  # noqa: F401
