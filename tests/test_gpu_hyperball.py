"""GPU parity of the Hyperball update (with and without the fixed-radius projection) against the
float64 oracle.

Tolerance, derived from the FP32 arithmetic of the update w' = fp32(w*fp32(1-lr*wd)) +
fp32(g*fp32(-lr/n)): each of the decay factor, the two products, the step coefficient and the sum
rounds once, so |w'_gpu - w'_64| <= 3 * 2^-24 * (|w|(1-lr*wd) + lr|g|/n); the test allows 2^-22 of
that magnitude.  The projection adds the rounding of its factor and of the product (and the
factor's dependence on the rounded w'), held to 2^-21 of the projected magnitude.  The reported
norms are fp32 roundings of fp64 sums: relative 2^-22 (gradient) and 2^-20 (weights).
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import oracle
import synth
from parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_step(w0, g, lr, wd, eps, radius, w_gpu, norms, what):
    ref, gnorm, wnorm = oracle.hyperball_step(w0, g.float().numpy() if torch.is_tensor(g) else g, lr, wd, eps, radius)
    g64 = (g.float().numpy() if torch.is_tensor(g) else g).astype(np.float64)
    n = max(gnorm, eps)
    mag = np.abs(w0.astype(np.float64)) * (1 - lr * wd) + lr * np.abs(g64) / n
    if radius > 0 and wnorm > 0:
        f = radius / wnorm
        lim = 2.0 ** -21 * f * mag + 2.0 ** -22 * np.abs(ref)
    else:
        lim = 2.0 ** -22 * mag
    got = w_gpu.astype(np.float64)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(lim, 1e-300)))
    assert np.all(err <= lim), f"{what}: max err / limit = {worst:.3f}"
    gn, wn = float(norms[0]), float(norms[1])
    assert abs(gn - gnorm) <= 2.0 ** -22 * gnorm, (what, gn, gnorm)
    assert abs(wn - wnorm) <= 2.0 ** -20 * wnorm + 1e-30, (what, wn, wnorm)
    say(f"{what}: max err / limit = {worst:.3f}, |g| = {gn:.6g}, |w| = {wn:.6g}")


@pytest.mark.parametrize("shape", [(128, 128), (300, 264), (1, 8), (1027, 520)])
@pytest.mark.parametrize("gdtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("radius", [0.0, 10.0])
def test_steps(shape, gdtype, radius):
    """Three steps in a row on one weight tensor, each checked against the oracle applied to the
    weights the previous GPU step left."""
    lr, wd, eps = 1e-2, 0.1, 1e-8
    w = synth.random_f32(shape, seed=shape[0] + 3, std=0.02).to(DEV)
    for step in range(3):
        g = synth.random_f32(shape, seed=100 * step + shape[1], std=1e-3).to(gdtype)
        w0 = w.cpu().numpy().copy()
        norms = fq.hyperball_step(w, g.to(DEV), lr, wd, eps, radius)
        torch.cuda.synchronize()
        _check_step(w0, g, lr, wd, eps, radius, w.cpu().numpy(), norms.cpu().numpy(),
                    f"hyperball {shape} {gdtype} R={radius} step {step}")


def test_pages_defaults_and_edge_cases():
    # the listing's defaults on a strided weight view (the padding columns must stay untouched)
    big = torch.full((64, 272), 9.0, dtype=torch.float32, device=DEV)
    w = big[:, :256]
    w.copy_(synth.random_f32((64, 256), seed=5, std=0.02).to(DEV))
    g = synth.random_bf16((64, 256), seed=6, std=1e-3)
    w0 = w.cpu().numpy().copy()
    norms = fq.hyperball_step(w, g.to(DEV))
    torch.cuda.synchronize()
    _check_step(w0, g, 1e-4, 0.1, 1e-8, 0.0, w.cpu().numpy(), norms.cpu().numpy(), "defaults, strided")
    assert torch.all(big[:, 256:] == 9.0)
    # an all-zero gradient: only the decay applies
    z = torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV)
    w1 = w.clone()
    fq.hyperball_step(w, z, 0.5, 0.1, 1e-8)
    torch.cuda.synchronize()
    assert torch.equal(w, w1 * np.float32(1 - 0.05))
    # a zero weight with a radius stays zero; no rows: nothing happens
    w2 = torch.zeros((8, 16), dtype=torch.float32, device=DEV)
    fq.hyperball_step(w2, torch.zeros((8, 16), dtype=torch.float32, device=DEV), 0.1, 0.1, 1e-8, radius=4.0)
    e = torch.empty((0, 16), dtype=torch.float32, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    fq.fp8bq_hyperball_step(e, e, 0.1, 0.1, 1e-8, 1.0, None, ws)
    torch.cuda.synchronize()
    assert torch.all(w2 == 0)


def test_full_size_weight():
    """The gate+up weight of the decoder block, 11264 x 2048 FP32 master weights, BF16 gradient,
    projected back to its initial radius."""
    w = synth.random_f32((11264, 2048), seed=11, std=0.02).to(DEV)
    radius = float(torch.linalg.vector_norm(w.double()).item())
    g = synth.random_bf16((11264, 2048), seed=12, std=1e-3)
    w0 = w.cpu().numpy().copy()
    norms = fq.hyperball_step(w, g.to(DEV), 1e-3, 0.1, 1e-8, radius)
    torch.cuda.synchronize()
    _check_step(w0, g, 1e-3, 0.1, 1e-8, radius, w.cpu().numpy(), norms.cpu().numpy(), "gate_up 11264x2048")


# ------------------------------------------------------------------------------------------
# several matrices per launch pair
# ------------------------------------------------------------------------------------------

def _batch_case(gdtype, n, seed):
    """n matrices of mixed shapes (ragged rows, one past the 1024-block cap), radius and norms
    mixed: with a radius and norms, norms only, neither."""
    shapes = [(128, 128), (300, 264), (1, 8), (1027, 520), (4100, 64), (256, 2048)]
    ws, gs, radii, want_norms = [], [], [], []
    for i in range(n):
        R, C = shapes[i % len(shapes)]
        ws.append(synth.random_f32((R, C), seed=seed + 2 * i, std=0.02).to(DEV))
        gs.append(synth.random_f32((R, C), seed=seed + 2 * i + 1, std=1e-3).to(gdtype).to(DEV))
        radii.append([0.0, 3.0, 0.0][i % 3])
        want_norms.append(i % 3 != 2)
    return ws, gs, radii, want_norms


@pytest.mark.parametrize("gdtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [1, 5, fq.MAX_HYPERBALL_JOBS])
def test_batch_matches_single_calls(gdtype, n):
    """Weights and norms of one batched call equal those of one call per matrix, bit for bit, and
    each matrix against the oracle."""
    lr, wd, eps = 1e-2, 0.1, 1e-8
    ws, gs, radii, want = _batch_case(gdtype, n, seed=700 + n)
    w_single = [w.clone() for w in ws]
    n_single = []
    for w, g, r, k in zip(w_single, gs, radii, want):
        norms = torch.zeros(2, dtype=torch.float32, device=DEV)
        ws_buf = torch.empty(max(fq.fp8bq_hyperball_workspace_size(*w.shape), 16), dtype=torch.uint8, device=DEV)
        fq.fp8bq_hyperball_step(w, g, lr, wd, eps, r, norms if k else None, ws_buf)
        n_single.append(norms)
    w0 = [w.cpu().numpy().copy() for w in ws]
    norms_b = torch.zeros((n, 2), dtype=torch.float32, device=DEV)
    wsb = torch.empty(fq.fp8bq_hyperball_batch_workspace_size(n), dtype=torch.uint8, device=DEV)
    fq.fp8bq_hyperball_step_batch([(w, g, r, norms_b[i] if k else None) for i, (w, g, r, k) in
                                   enumerate(zip(ws, gs, radii, want))], lr, wd, eps, wsb)
    torch.cuda.synchronize()
    for i in range(n):
        assert torch.equal(ws[i], w_single[i]), f"weights of job {i}"
        assert torch.equal(norms_b[i], n_single[i]), f"norms of job {i}"
        if want[i]:
            _check_step(w0[i], gs[i].cpu(), lr, wd, eps, radii[i], ws[i].cpu().numpy(), norms_b[i].cpu().numpy(),
                        f"batch {n} job {i} {tuple(ws[i].shape)} R={radii[i]}")


def test_batch_helper_over_the_job_limit():
    """hyperball_step_batch splits more than MAX_HYPERBALL_JOBS matrices over several launch pairs."""
    n = fq.MAX_HYPERBALL_JOBS + 3
    ws, gs, _, _ = _batch_case(torch.bfloat16, n, seed=900)
    ref = [w.clone() for w in ws]
    ref_norms = torch.stack([fq.hyperball_step(w, g, 1e-3, 0.1, 1e-8, 2.0) for w, g in zip(ref, gs)])
    norms = fq.hyperball_step_batch(ws, gs, 1e-3, 0.1, 1e-8, radii=[2.0] * n)
    torch.cuda.synchronize()
    assert torch.equal(norms, ref_norms)
    assert all(torch.equal(a, b) for a, b in zip(ws, ref))


def test_batch_error_enqueues_nothing():
    """A batch whose second job writes onto the first job's gradient fails as a whole: nothing is
    written, the valid job included."""
    w0 = torch.full((256, 256), 1.5, dtype=torch.float32, device=DEV)
    g0 = torch.full((256, 256), 0.25, dtype=torch.float32, device=DEV)
    w1 = g0[:128]  # job 1's weights are job 0's gradient
    g1 = torch.ones((128, 256), dtype=torch.float32, device=DEV)
    wsb = torch.empty(fq.fp8bq_hyperball_batch_workspace_size(2), dtype=torch.uint8, device=DEV)
    with pytest.raises(fq.Fp8bqError) as e:
        fq.fp8bq_hyperball_step_batch([(w0, g0, 0.0, None), (w1, g1, 0.0, None)], 1e-2, 0.1, 1e-8, wsb)
    assert e.value.status == 10  # FP8BQ_ERR_OVERLAP
    torch.cuda.synchronize()
    assert bool((w0 == 1.5).all()) and bool((g0 == 0.25).all())
