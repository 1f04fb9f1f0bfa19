"""GPU parity of the three quantize kernels against the CPU oracle: codes and FP32 scales must be
bit-identical, compared in logical (row, group) coordinates.

Small cases span several tiles and ragged tails; the full-size workloads are compared in full where
the oracle is quick (the 8192x2048 activation and weight), otherwise on sampled rows (1x128 groups
are independent per row) or sampled columns (128x1 groups are independent per column).
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import oracle
import synth
from parity import FP, f32_bits, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = [oracle.E4M3, oracle.E5M2]


def gpu_1x128(x, fmt):
    q, s = fq.quantize_act_1x128(x.to(DEV), FP[fmt])
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy().T  # s -> logical [R, C/128]


def gpu_128x1(x, fmt):
    qt, st = fq.quantize_act_128x1(x.to(DEV), FP[fmt])
    torch.cuda.synchronize()
    return qt.cpu().numpy().T, st.cpu().numpy()  # codes back in x's orientation


def gpu_w(w, fmt):
    q, s = fq.quantize_weight_128x128(w.to(DEV), FP[fmt])
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def same(got, exp, what):
    qg, sg = got
    qe, se = exp
    assert qg.shape == qe.shape and sg.shape == se.shape, what
    bad = np.argwhere(qg != qe)
    assert bad.size == 0, f"{what}: {len(bad)} code mismatches, first at {bad[:3].tolist()}"
    sb = np.argwhere(f32_bits(sg) != f32_bits(se))
    assert sb.size == 0, f"{what}: {len(sb)} scale mismatches, first at {sb[:3].tolist()}"


# ------------------------------------------------------------------------------------------
# the hardware FP8 conversion, driven through the 1x128 quantizer with scale exactly 1
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_every_decision_point(fmt):
    """Each row holds fmt_max (so s = 1 and y = x exactly) and 127 probe values; probes cover every
    fp32 exponent up to the maximum x every top-11 mantissa pattern x 4 low-bit patterns, both
    signs, plus every midpoint between adjacent codes and its two neighbours."""
    m = np.float32(oracle.fmt_max(fmt))
    emax = 127 + int(np.floor(np.log2(float(m))))
    exps = np.arange(0, emax + 1, dtype=np.uint32)
    top = np.arange(1 << 11, dtype=np.uint32) << np.uint32(12)
    low = np.array([0, 1, 0x7FF, 0x800], dtype=np.uint32)
    bits = ((exps[:, None, None] << np.uint32(23)) | top[None, :, None] | low[None, None, :]).reshape(-1)
    y = bits.view(np.float32)
    y = y[np.abs(y) <= m]
    tab = oracle.decode_table(fmt)
    n = int(np.isfinite(tab[:128]).sum())
    mids = np.array([0.5 * (tab[c] + tab[c + 1]) for c in range(n - 1)], np.float32)
    extra = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    y = np.concatenate([y, -y, extra, -extra, np.array([0.0, -0.0], np.float32)])
    rows = (y.size + 126) // 127
    pad = np.zeros(rows * 127, np.float32)
    pad[:y.size] = y
    x = np.empty((rows, 128), np.float32)
    x[:, 0] = m
    x[:, 1:] = pad.reshape(rows, 127)
    say(f"encoder sweep {fmt}: {x.size} values")
    qg, sg = gpu_1x128(torch.from_numpy(x), fmt)
    assert np.all(sg == 1.0)
    exp = oracle.encode(x, fmt)
    bad = np.argwhere(qg != exp)
    assert bad.size == 0, (bad[:3], x[tuple(bad[0])], qg[tuple(bad[0])], exp[tuple(bad[0])])


# ------------------------------------------------------------------------------------------
# tiny workload (FP32 inputs)
# ------------------------------------------------------------------------------------------

def test_tiny_workload_all_quantizers():
    c = synth.tiny_check()
    A, W, dY = c["A"], c["W"], c["dY"]
    same(gpu_1x128(A, oracle.E4M3), oracle.quant_act_1x128(A.numpy(), oracle.E4M3), "A 1x128")
    same(gpu_w(W, oracle.E4M3), oracle.quant_weight_128x128(W.numpy(), oracle.E4M3), "W 128x128")
    for fmt in FMTS:
        same(gpu_1x128(dY, fmt), oracle.quant_act_1x128(dY.numpy(), fmt), f"dY 1x128 {fmt}")
        same(gpu_128x1(dY, fmt), oracle.quant_act_128x1(dY.numpy(), fmt), f"dY 128x1 {fmt}")
        same(gpu_128x1(A, fmt), oracle.quant_act_128x1(A.numpy(), fmt), f"A 128x1 {fmt}")


# ------------------------------------------------------------------------------------------
# ragged and strided shapes
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("R", [1, 5, 63, 64, 65, 200, 1000])
def test_1x128_ragged_rows(fmt, R):
    x = synth.random_bf16((R, 384), seed=100 + R, outliers=True)
    same(gpu_1x128(x, fmt), oracle.quant_act_1x128(x.float().numpy(), fmt), f"1x128 R={R}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(128, 8), (256, 72), (384, 200), (128, 1000), (640, 64)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_128x1_shapes(fmt, shape, dt):
    x = synth.random_bf16(shape, seed=200 + shape[1], outliers=True)
    if dt == "f32":
        x = synth.random_f32(shape, seed=300 + shape[1])
    same(gpu_128x1(x, fmt), oracle.quant_act_128x1(x.float().numpy(), fmt), f"128x1 {shape} {dt}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(128, 128), (384, 256), (256, 640)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_weight_shapes(fmt, shape, dt):
    w = synth.random_bf16(shape, seed=400 + shape[1], std=0.02)
    if dt == "f32":
        w = synth.random_f32(shape, seed=500 + shape[1], std=0.02)
    same(gpu_w(w, fmt), oracle.quant_weight_128x128(w.float().numpy(), fmt), f"weight {shape} {dt}")


def test_strided_views():
    big = synth.random_bf16((300, 512), seed=7, outliers=True).to(DEV)
    x = big[:, 64:448]  # R=300, C=384, ldx=512
    q = torch.zeros((300, 400), dtype=torch.uint8, device=DEV)[:, :384]
    s = torch.zeros((3, 304 + 8), dtype=torch.float32, device=DEV)[:, :300]
    fq.fp8bq_quantize_act_1x128(x, fq.E4M3, q, s)
    torch.cuda.synchronize()
    same((q.cpu().numpy(), s.cpu().numpy().T), oracle.quant_act_1x128(x.float().cpu().numpy(), oracle.E4M3),
         "strided 1x128")
    x2 = big[:256, 8:200]  # R=256, C=192
    qt = torch.zeros((192, 272), dtype=torch.uint8, device=DEV)[:, :256]
    st = torch.zeros((2, 200), dtype=torch.float32, device=DEV)[:, :192]
    fq.fp8bq_quantize_act_128x1(x2, fq.E5M2, qt, st)
    torch.cuda.synchronize()
    same((qt.cpu().numpy().T, st.cpu().numpy()), oracle.quant_act_128x1(x2.float().cpu().numpy(), oracle.E5M2),
         "strided 128x1")
    w = big[:256, 128:384]
    qw = torch.zeros((256, 272), dtype=torch.uint8, device=DEV)[:, :256]
    sw = torch.zeros((2, 3), dtype=torch.float32, device=DEV)[:, :2]
    fq.fp8bq_quantize_weight_128x128(w, fq.E4M3, qw, sw)
    torch.cuda.synchronize()
    same((qw.cpu().numpy(), sw.cpu().numpy()), oracle.quant_weight_128x128(w.float().cpu().numpy(), oracle.E4M3),
         "strided weight")


def _edge_matrix():
    """256x256 BF16 with degenerate groups: zeros, negative zeros, floor-scale groups, BF16
    subnormals, the BF16 maximum, single spikes, exact powers of two and ties after scaling."""
    x = synth.random_bf16((256, 256), seed=77).float().numpy()
    x[0, :128] = 0.0
    x[1, :128] = -0.0
    x[2, :128] = np.float32(1e-13)
    x[3, :128] = np.float32(2.0 ** -130)  # BF16 subnormal
    x[4, :128] = np.float32(3.3895313892515355e38)  # BF16 max
    x[4, 5] = -x[4, 5]
    x[5, :128] = 0.0
    x[5, 77] = -5.0
    x[6, :128] = np.float32(448.0) * np.float32(2.0) ** np.arange(-64, 64, dtype=np.float32) / np.float32(2 ** 20)
    x[7, :128] = np.float32(896.0)
    x[7, 1:128] = np.float32(3 * 2 ** -9)  # 3*2^-10 after s = 2: E4M3 tie -> even
    x[8:, 128:] *= np.float32(1e-30)
    x[:128, 0] = 0.0  # a zero 128x1 group in column 0
    x[128:, 1] = -0.0
    return torch.from_numpy(x).to(torch.bfloat16)


@pytest.mark.parametrize("fmt", FMTS)
def test_edge_values(fmt):
    x = _edge_matrix()
    xf = x.float().numpy()
    same(gpu_1x128(x, fmt), oracle.quant_act_1x128(xf, fmt), "edge 1x128")
    same(gpu_128x1(x, fmt), oracle.quant_act_128x1(xf, fmt), "edge 128x1")
    same(gpu_w(x, fmt), oracle.quant_weight_128x128(xf, fmt), "edge 128x128")


def test_deterministic():
    x = synth.random_bf16((1024, 2048), seed=9, outliers=True).to(DEV)
    a = fq.quantize_act_1x128(x)
    b = fq.quantize_act_1x128(x)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------------------------------
# full-size workloads
# ------------------------------------------------------------------------------------------

def test_single_linear_full():
    c = synth.single_linear()
    say("8192x2048 activation and weight, full comparison")
    same(gpu_1x128(c["X"], oracle.E4M3), oracle.quant_act_1x128(c["X"].float().numpy(), oracle.E4M3), "X 1x128")
    same(gpu_w(c["W"], oracle.E4M3), oracle.quant_weight_128x128(c["W"].float().numpy(), oracle.E4M3), "W")


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(n, size=min(k, n), replace=False))
    idx[0], idx[-1] = 0, n - 1
    return np.unique(idx)


def _check_act_sampled(x, fmt, what, seed):
    """1x128 on sampled rows, 128x1 on sampled columns, of the full GPU result."""
    R, C = x.shape
    rows = _sample(R, 256, seed)
    cols = _sample(C, 64, seed + 1)
    xd = x.to(DEV)
    q, s = fq.quantize_act_1x128(xd, FP[fmt])
    qt, st = fq.quantize_act_128x1(xd, FP[fmt])
    torch.cuda.synchronize()
    xs = x[rows].float().numpy()
    same((q.cpu().numpy()[rows], s.cpu().numpy().T[rows]), oracle.quant_act_1x128(xs, fmt), what + " 1x128")
    xc = np.ascontiguousarray(x[:, cols].float().numpy())
    same((qt.cpu().numpy()[cols].T, st.cpu().numpy()[:, cols]), oracle.quant_act_128x1(xc, fmt), what + " 128x1")


@pytest.mark.parametrize("name", [n for n, _, _ in synth.DECODER_LINEARS])
def test_decoder_block_sampled(name):
    say(f"decoder block linear {name}")
    c = synth.decoder_linear(name)
    _check_act_sampled(c["X"], oracle.E4M3, f"{name} X", 1)
    _check_act_sampled(c["dY"], oracle.E4M3, f"{name} dY", 2)
    same(gpu_w(c["W"], oracle.E4M3), oracle.quant_weight_128x128(c["W"].float().numpy(), oracle.E4M3), f"{name} W")


def test_sweep_activations_sampled():
    for M in synth.SWEEP_M:
        x = synth.sweep_x(M)
        rows = _sample(M, 128, M)
        q, s = gpu_1x128(x, oracle.E4M3)
        same((q[rows], s[rows]), oracle.quant_act_1x128(x[rows].float().numpy(), oracle.E4M3), f"sweep M={M}")
    w = synth.sweep_weight()
    same(gpu_w(w, oracle.E4M3), oracle.quant_weight_128x128(w.float().numpy(), oracle.E4M3), "sweep W")


def test_heavy_tailed_gradients_sampled():
    c = synth.heavy_tailed()
    _check_act_sampled(c["dY"], oracle.E5M2, "dY E5M2", 3)
    _check_act_sampled(c["dY"], oracle.E4M3, "dY E4M3", 4)
    _check_act_sampled(c["X"], oracle.E4M3, "X", 5)
    same(gpu_w(c["W"], oracle.E4M3), oracle.quant_weight_128x128(c["W"].float().numpy(), oracle.E4M3), "W")


# ------------------------------------------------------------------------------------------
# both activation layouts from one pass
# ------------------------------------------------------------------------------------------

def gpu_dual(x, fr, fc):
    q, s, qt, st = fq.quantize_act_dual(x.to(DEV), FP[fr], FP[fc])
    torch.cuda.synchronize()
    return (q.cpu().numpy(), s.cpu().numpy().T), (qt.cpu().numpy().T, st.cpu().numpy())


@pytest.mark.parametrize("fr,fc", [(oracle.E4M3, oracle.E4M3), (oracle.E5M2, oracle.E4M3),
                                   (oracle.E4M3, oracle.E5M2), (oracle.E5M2, oracle.E5M2)])
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (640, 256)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_dual_shapes(fr, fc, shape, dt):
    R, C = shape
    x = synth.random_bf16(shape, seed=R + C, outliers=True) if dt == "bf16" else synth.random_f32(shape, seed=R + C)
    xf = x.float().numpy()
    rows, cols = gpu_dual(x, fr, fc)
    same(rows, oracle.quant_act_1x128(xf, fr), f"dual 1x128 {shape} {dt}")
    same(cols, oracle.quant_act_128x1(xf, fc), f"dual 128x1 {shape} {dt}")


def test_dual_edge_values_and_strides():
    x = _edge_matrix()
    xf = x.float().numpy()
    for fr, fc in [(oracle.E4M3, oracle.E5M2), (oracle.E5M2, oracle.E4M3)]:
        rows, cols = gpu_dual(x, fr, fc)
        same(rows, oracle.quant_act_1x128(xf, fr), "edge dual 1x128")
        same(cols, oracle.quant_act_128x1(xf, fc), "edge dual 128x1")
    big = synth.random_bf16((384, 512), seed=8, outliers=True).to(DEV)
    xs = big[:256, 128:384]  # R=256, C=256, ldx=512
    q = torch.zeros((256, 272), dtype=torch.uint8, device=DEV)[:, :256]
    s = torch.zeros((2, 264), dtype=torch.float32, device=DEV)[:, :256]
    qt = torch.zeros((256, 288), dtype=torch.uint8, device=DEV)[:, :256]
    st = torch.zeros((2, 260), dtype=torch.float32, device=DEV)[:, :256]
    fq.fp8bq_quantize_act_dual(xs, fq.E4M3, q, s, fq.E5M2, qt, st)
    torch.cuda.synchronize()
    xsf = xs.float().cpu().numpy()
    same((q.cpu().numpy(), s.cpu().numpy().T), oracle.quant_act_1x128(xsf, oracle.E4M3), "strided dual 1x128")
    same((qt.cpu().numpy().T, st.cpu().numpy()), oracle.quant_act_128x1(xsf, oracle.E5M2), "strided dual 128x1")


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_dual_decoder_block_sampled(name):
    """Full-size decoder-block activations: rows and columns sampled as in the single-layout checks."""
    c = synth.decoder_linear(name)
    for key, fr, fc, seed in [("X", oracle.E4M3, oracle.E4M3, 11), ("dY", oracle.E5M2, oracle.E4M3, 12)]:
        x = c[key]
        R, C = x.shape
        say(f"dual {name} {key} {R}x{C}")
        q, s, qt, st = fq.quantize_act_dual(x.to(DEV), FP[fr], FP[fc])
        torch.cuda.synchronize()
        rows = _sample(R, 256, seed)
        cols = _sample(C, 64, seed + 1)
        same((q.cpu().numpy()[rows], s.cpu().numpy().T[rows]), oracle.quant_act_1x128(x[rows].float().numpy(), fr),
             f"dual {name} {key} 1x128")
        xc = np.ascontiguousarray(x[:, cols].float().numpy())
        same((qt.cpu().numpy()[cols].T, st.cpu().numpy()[:, cols]), oracle.quant_act_128x1(xc, fc),
             f"dual {name} {key} 128x1")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(128, 128), (384, 256), (256, 640)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_weight_dual_shapes(fmt, shape, dt):
    """Weight codes, scales and the transposed codes from one pass: all bit-identical to the oracle."""
    N, K = shape
    w = synth.random_bf16(shape, seed=N + 2 * K, std=0.02) if dt == "bf16" else synth.random_f32(shape, seed=N + 2 * K)
    q, s, qt = fq.quantize_weight_dual(w.to(DEV), FP[fmt])
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_weight_128x128(w.float().numpy(), fmt)
    same((q.cpu().numpy(), s.cpu().numpy()), (oq, os_), f"weight dual {shape} {dt}")
    assert np.array_equal(qt.cpu().numpy(), oq.T), "transposed codes"


def test_weight_dual_full_size_and_edges():
    c = synth.decoder_linear("gate_up")
    W = c["W"]
    q, s, qt = fq.quantize_weight_dual(W.to(DEV), fq.E4M3)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_weight_128x128(W.float().numpy(), oracle.E4M3)
    same((q.cpu().numpy(), s.cpu().numpy()), (oq, os_), "gate_up W dual")
    assert np.array_equal(qt.cpu().numpy(), oq.T)
    x = _edge_matrix()
    q, s, qt = fq.quantize_weight_dual(x.to(DEV), fq.E5M2)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_weight_128x128(x.float().numpy(), oracle.E5M2)
    same((q.cpu().numpy(), s.cpu().numpy()), (oq, os_), "edge weight dual")
    assert np.array_equal(qt.cpu().numpy(), oq.T)


# ------------------------------------------------------------------------------------------
# several weights in one launch
# ------------------------------------------------------------------------------------------

def _padded_job(w, fmt_pad=(16, 4, 32)):
    """Outputs for w in padded layouts (row strides beyond the row length), as views."""
    N, K = w.shape
    pq, ps, pqt = fmt_pad
    q = torch.empty((N, K + pq), dtype=torch.uint8, device=DEV)[:, :K]
    s = torch.empty((N // 128, K // 128 + ps), dtype=torch.float32, device=DEV)[:, :K // 128]
    qt = torch.empty((K, N + pqt), dtype=torch.uint8, device=DEV)[:, :N]
    return q, s, qt


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_weights_batch_matches_single_and_oracle(fmt, dt):
    """One launch over weights of mixed shapes (one empty, one a strided view, one with padded
    outputs): every job's codes, scales and transposed codes equal the single-weight kernel's and
    the oracle's, bit for bit."""
    gen = (lambda shape, seed: synth.random_bf16(shape, seed=seed, std=0.02)) if dt == "bf16" else \
        (lambda shape, seed: synth.random_f32(shape, seed=seed))
    big = gen((256, 1024), 31).to(DEV)
    ws = [gen((128, 128), 11).to(DEV), gen((384, 256), 12).to(DEV), gen((0, 256), 13).to(DEV),
          big[:, 128:512], gen((256, 640), 14).to(DEV)]
    outs = []
    for i, w in enumerate(ws):
        N, K = w.shape
        if i == 4:
            outs.append(_padded_job(w))
        else:
            outs.append((torch.empty((N, K), dtype=torch.uint8, device=DEV),
                         torch.empty((N // 128, K // 128), dtype=torch.float32, device=DEV),
                         torch.empty((K, N), dtype=torch.uint8, device=DEV)))
    fq.fp8bq_quantize_weights_dual([(w,) + o for w, o in zip(ws, outs)], FP[fmt])
    torch.cuda.synchronize()
    for i, (w, (q, s, qt)) in enumerate(zip(ws, outs)):
        if w.shape[0] == 0:
            continue
        q1, s1, qt1 = fq.quantize_weight_dual(w, FP[fmt])
        torch.cuda.synchronize()
        assert torch.equal(q, q1) and torch.equal(qt, qt1), f"job {i}: codes differ from the single-weight call"
        assert np.array_equal(f32_bits(s.cpu().numpy()), f32_bits(s1.cpu().numpy())), f"job {i}: scales"
        oq, os_ = oracle.quant_weight_128x128(w.float().cpu().numpy(), fmt)
        same((q.cpu().numpy(), s.cpu().numpy()), (oq, os_), f"batched weight job {i} {tuple(w.shape)} {dt}")
        assert np.array_equal(qt.cpu().numpy(), oq.T), f"job {i}: transposed codes"
    say(f"batched weight quantization ({fmt}, {dt}): {len(ws)} jobs bit-identical to single calls and the oracle")


def test_weights_batch_decoder_block_and_many():
    """The decoder block's four weights in one launch (bit-identical to four single-weight launches,
    and to the oracle for two of them); then 20 small weights, which the helper splits into two
    launches of at most 16."""
    ws = [synth.decoder_linear(n)["W"] for n, _, _ in synth.DECODER_LINEARS]
    wd = [w.to(DEV) for w in ws]
    outs = fq.quantize_weights_dual(wd, fq.E4M3)
    singles = [fq.quantize_weight_dual(w, fq.E4M3) for w in wd]
    torch.cuda.synchronize()
    for (n, _, _), o, s1 in zip(synth.DECODER_LINEARS, outs, singles):
        for a, b in zip(o, s1):
            assert torch.equal(a, b), f"{n}: batched and single-weight outputs differ"
    for i in (1, 3):
        oq, os_ = oracle.quant_weight_128x128(ws[i].float().numpy(), oracle.E4M3)
        same((outs[i][0].cpu().numpy(), outs[i][1].cpu().numpy()), (oq, os_), f"{synth.DECODER_LINEARS[i][0]} W")
        assert np.array_equal(outs[i][2].cpu().numpy(), oq.T)
    many = [synth.random_bf16((128 * (1 + i % 3), 128 * (1 + i % 2)), seed=900 + i, std=0.5).to(DEV)
            for i in range(20)]
    outs = fq.quantize_weights_dual(many, fq.E5M2)
    torch.cuda.synchronize()
    for i, (w, (q, s, qt)) in enumerate(zip(many, outs)):
        oq, os_ = oracle.quant_weight_128x128(w.float().cpu().numpy(), oracle.E5M2)
        same((q.cpu().numpy(), s.cpu().numpy()), (oq, os_), f"small weight {i}")
        assert np.array_equal(qt.cpu().numpy(), oq.T)


def test_weights_batch_error_enqueues_nothing():
    """A batch with one bad job fails as a whole: the status is returned and no job's outputs are
    written, the valid ones included."""
    w0 = synth.random_bf16((256, 256), seed=41, std=0.1).to(DEV)
    w1 = synth.random_bf16((128, 256), seed=42, std=0.1).to(DEV)
    q0 = torch.full((256, 256), 0xA5, dtype=torch.uint8, device=DEV)
    s0 = torch.full((2, 2), -1.0, dtype=torch.float32, device=DEV)
    qt0 = torch.full((256, 256), 0x5A, dtype=torch.uint8, device=DEV)
    q1 = torch.empty((128, 256), dtype=torch.uint8, device=DEV)
    s1 = torch.empty((1, 2), dtype=torch.float32, device=DEV)
    bad_qt1 = q0[:, :128]  # job 1's W^T codes [256, 128] would land on job 0's codes
    with pytest.raises(fq.Fp8bqError) as e:
        fq.fp8bq_quantize_weights_dual([(w0, q0, s0, qt0), (w1, q1, s1, bad_qt1)], fq.E4M3)
    assert e.value.status == 10  # FP8BQ_ERR_OVERLAP
    qt1 = torch.empty((200, 128), dtype=torch.uint8, device=DEV)
    # tensors of the shapes the binding derives from K = 200, so the call reaches the library's check
    with pytest.raises(fq.Fp8bqError) as e:
        fq.fp8bq_quantize_weights_dual([(w0, q0, s0, qt0), (w1[:, :200], q1[:, :200], s1[:, :1], qt1)], fq.E4M3)
    assert e.value.status == 2  # FP8BQ_ERR_SHAPE: K = 200
    torch.cuda.synchronize()
    assert bool((q0 == 0xA5).all()) and bool((qt0 == 0x5A).all()) and bool((s0 == -1.0).all())


# ------------------------------------------------------------------------------------------
# group amax whose quotient rounds to just above the format maximum
# ------------------------------------------------------------------------------------------

def _over_max_amax(fmt, dt):
    """Positive values a (every BF16 one, or a log-uniform FP32 sample) for which fp32(a / s), with
    s = max(fp32(a / fmt_max), 1e-12), is above fmt_max: a group whose amax is a then divides a to
    fmt_max + 1 ulp, and its code must still be the fmt_max code."""
    m = np.float32(oracle.fmt_max(fmt))
    if dt == "bf16":
        a = torch.arange(1, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float().numpy()
    else:
        rng = np.random.default_rng(23)
        a = np.exp(rng.uniform(-60.0, 60.0, 400_000)).astype(np.float32)
    s = np.maximum(a / m, np.float32(1e-12)).astype(np.float32)
    q = (a / s).astype(np.float32)
    assert np.all(q <= np.nextafter(m, np.float32(np.inf)))  # never more than one ulp above
    return a[q > m]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_group_amax_quotient_just_above_the_maximum(fmt, dt):
    """About one group in twelve has an amax whose quotient rounds above fmt_max.  Rows of +a and -a
    (each such a) plus smaller values, so that rows, columns and 128x128 tiles all have such an amax:
    codes and scales of every quantizer bit-identical to the oracle, with the fmt_max codes present."""
    a = _over_max_amax(fmt, dt)
    assert a.size > 1000
    R = 128 * ((a.size + 127) // 128)
    amax = np.resize(a, R).astype(np.float32)
    rng = np.random.default_rng(29)
    x = (rng.uniform(-1.0, 1.0, (R, 128)).astype(np.float32) * amax[:, None]).astype(np.float32)
    r = np.arange(R)
    x[r, r % 128] = amax
    x[r, (r + 1) % 128] = -amax
    xt = torch.from_numpy(x).to(torch.bfloat16) if dt == "bf16" else torch.from_numpy(x)
    xf = xt.float().numpy()
    assert np.array_equal(np.abs(xf).max(axis=1), amax)
    say(f"over-max quotients {fmt} {dt}: {a.size} amax values, {R} rows")
    top = oracle.encode(np.array([oracle.fmt_max(fmt), -oracle.fmt_max(fmt)], np.float32), fmt)
    e_rows, e_cols = oracle.quant_act_1x128(xf, fmt), oracle.quant_act_128x1(xf, fmt)
    g_rows = gpu_1x128(xt, fmt)
    assert np.all((g_rows[0] == top[0]).sum(axis=1) >= 1) and np.all((g_rows[0] == top[1]).sum(axis=1) >= 1)
    same(g_rows, e_rows, "1x128")
    same(gpu_128x1(xt, fmt), e_cols, "128x1")
    d_rows, d_cols = gpu_dual(xt, fmt, fmt)
    same(d_rows, e_rows, "dual 1x128")
    same(d_cols, e_cols, "dual 128x1")
    e_w = oracle.quant_weight_128x128(xf, fmt)
    same(gpu_w(xt, fmt), e_w, "128x128")
    q, s, qt = fq.quantize_weight_dual(xt.to(DEV), FP[fmt])
    torch.cuda.synchronize()
    same((q.cpu().numpy(), s.cpu().numpy()), e_w, "128x128 dual")
    assert np.array_equal(qt.cpu().numpy(), e_w[0].T), "transposed weight codes"
