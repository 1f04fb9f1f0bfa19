"""Hyperball normalized update of one weight matrix, with the optional
fixed-radius projection.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* [HL] section "Hyperball 优化：让 FP8 训练不爆炸", the ``HyperballSGD``
  listing: the gradient's direction is kept and its magnitude dropped.  Per
  parameter, n = max(||g||_2, eps) (the norm clamped from below); the weight
  first decays, w <- w * (1 - lr * wd) (decoupled weight decay), and then
  moves by -lr along g / n.  Defaults lr = 1e-4, wd = 0.1, eps = 1e-8.
* [XZY] paragraph on MuonH and [APD] "方法关键点" (MuonH bullet): after the
  update the weight is projected back onto a fixed radius, which fixes both
  the update's norm and the weight's norm.  Here that is w <- R * w / ||w||_F
  for a caller-given radius R > 0 (R = 0: no projection).  A zero weight has
  no direction and is left as it is.  Muon's orthogonalization of the update
  is not on the pages and is not part of this step.
* [HL] section "调试 FP8 训练的关键步骤": print the gradient norm, so the step
  also reports ||g||_2 (before the clamp).

Everything is float64: the method's result is defined by these formulas, and
the GPU's FP32 arithmetic is held to a tolerance around it.
"""

import numpy as np


def hyperball_step(w, g, lr, weight_decay, eps, radius=0.0):
    """w, g: arrays of one shape (w float32 master weights, g BF16- or FP32-valued gradient).

    Returns (new weights float64, ||g||_2 float64, ||w after the update||_2 float64).
    """
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if w.shape != g.shape:
        raise ValueError("w and g must have one shape")
    gnorm = float(np.sqrt(np.sum(g * g)))
    n = max(gnorm, float(eps))
    w_new = w * (1.0 - lr * weight_decay) - lr * (g / n)
    wnorm = float(np.sqrt(np.sum(w_new * w_new)))
    if radius > 0.0 and wnorm > 0.0:
        w_new = w_new * (radius / wnorm)
    return w_new, gnorm, wnorm
