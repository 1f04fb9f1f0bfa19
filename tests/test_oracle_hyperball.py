"""Pins for the oracle's Hyperball step (CPU only).

What pins it, independent of the code under test:
* the pages' HyperballSGD listing run as a torch optimizer on a float64 parameter (its clamp of the
  norm, decoupled decay, then the move along the normalized gradient);
* closed forms: a one-hot gradient moves exactly one weight by lr; lr = 0 or wd = 0 special cases;
  a gradient below eps is divided by eps, not by its norm;
* invariants: the move (after the decay) has norm exactly lr whenever ||g|| >= eps; the projection
  gives norm R and keeps the direction; a zero weight is left alone.
"""

import numpy as np
import pytest
import torch

from oracle import hyperball_step


def _listing_step(w, g, lr, wd, eps):
    """The pages' HyperballSGD.step for one parameter, written as a torch optimizer over float64."""

    class Hyperball(torch.optim.Optimizer):
        def __init__(self, params):
            super().__init__(params, dict(lr=lr, weight_decay=wd, eps=eps))

        @torch.no_grad()
        def step(self):
            for group in self.param_groups:
                for p in group["params"]:
                    n = torch.norm(p.grad).clamp(min=group["eps"])
                    p.mul_(1.0 - group["lr"] * group["weight_decay"])
                    p.add_(p.grad / n, alpha=-group["lr"])

    p = torch.nn.Parameter(torch.from_numpy(np.array(w, dtype=np.float64)))
    p.grad = torch.from_numpy(np.array(g, dtype=np.float64))
    Hyperball([p]).step()
    return p.detach().numpy()


@pytest.mark.parametrize("lr,wd,eps", [(1e-4, 0.1, 1e-8), (3e-2, 0.0, 1e-8), (1e-3, 0.5, 10.0)])
def test_matches_the_listing(lr, wd, eps):
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 96)) * 0.02).astype(np.float32)
    g = (rng.standard_normal((64, 96)) * 1e-3).astype(np.float32)
    got, gnorm, _ = hyperball_step(w, g, lr, wd, eps)
    want = _listing_step(w, g, lr, wd, eps)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-18)
    assert gnorm == pytest.approx(np.linalg.norm(g.astype(np.float64)), rel=1e-14)


def test_one_hot_gradient():
    w = np.full((4, 8), 0.5, np.float32)
    g = np.zeros((4, 8), np.float32)
    g[2, 5] = -3.0
    got, gnorm, _ = hyperball_step(w, g, 0.01, 0.1, 1e-8)
    want = np.full((4, 8), 0.5 * (1 - 0.001))
    want[2, 5] += 0.01  # -lr * (-3 / 3)
    assert gnorm == 3.0
    assert np.allclose(got, want, rtol=0, atol=1e-16)


def test_no_learning_rate_and_no_decay():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((8, 16)).astype(np.float32)
    g = rng.standard_normal((8, 16)).astype(np.float32)
    assert np.array_equal(hyperball_step(w, g, 0.0, 0.1, 1e-8)[0], w.astype(np.float64))
    got, _, _ = hyperball_step(w, g, 0.1, 0.0, 1e-8)
    g64 = g.astype(np.float64)
    assert np.allclose(got - w, -0.1 * g64 / np.linalg.norm(g64), rtol=0, atol=1e-15)


def test_small_gradient_divides_by_eps():
    w = np.zeros((2, 8), np.float32)
    g = np.zeros((2, 8), np.float32)
    g[0, 0] = 2.0 ** -30
    got, gnorm, _ = hyperball_step(w, g, 1.0, 0.0, 2.0 ** -26)
    assert got[0, 0] == -1.0 / 16  # -lr * 2^-30 / 2^-26, not -lr * sign
    assert gnorm == 2.0 ** -30


def test_move_has_norm_lr():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((32, 64)).astype(np.float32)
    g = rng.standard_normal((32, 64)).astype(np.float32) * 7
    lr, wd = 0.02, 0.1
    got, _, _ = hyperball_step(w, g, lr, wd, 1e-8)
    move = got - w.astype(np.float64) * (1 - lr * wd)
    assert np.linalg.norm(move) == pytest.approx(lr, rel=1e-13)


@pytest.mark.parametrize("radius", [1.0, 37.5])
def test_projection_to_the_radius(radius):
    rng = np.random.default_rng(4)
    w = rng.standard_normal((16, 32)).astype(np.float32)
    g = rng.standard_normal((16, 32)).astype(np.float32)
    free, _, wnorm = hyperball_step(w, g, 0.05, 0.1, 1e-8)
    proj, _, wnorm2 = hyperball_step(w, g, 0.05, 0.1, 1e-8, radius=radius)
    assert wnorm == pytest.approx(np.linalg.norm(free), rel=1e-14) and wnorm2 == wnorm
    assert np.linalg.norm(proj) == pytest.approx(radius, rel=1e-14)
    assert np.allclose(proj / radius, free / np.linalg.norm(free), rtol=0, atol=1e-15)


def test_zero_weight_is_not_projected():
    w = np.zeros((2, 8), np.float32)
    g = np.zeros((2, 8), np.float32)
    got, gnorm, wnorm = hyperball_step(w, g, 0.1, 0.1, 1e-8, radius=5.0)
    assert gnorm == 0.0 and wnorm == 0.0 and np.all(got == 0.0)
