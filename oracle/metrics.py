"""Error metrics, accumulated in float64. Test infrastructure only."""

import numpy as np


def mse(x_hat, x):
    """Mean squared error (the metric [EQuARX] Fig. 7 plots)."""
    d = np.asarray(x_hat, np.float64) - np.asarray(x, np.float64)
    return float(np.mean(d * d)) if d.size else 0.0


def rel_mse(x_hat, x):
    """sum (x_hat - x)^2 / sum x^2."""
    x = np.asarray(x, np.float64)
    d = np.asarray(x_hat, np.float64) - x
    den = float(np.sum(x * x))
    return float(np.sum(d * d)) / den if den > 0 else float(np.sum(d * d))


def rel_l2(a, b):
    """||a - b||_2 / ||b||_2."""
    b = np.asarray(b, np.float64)
    d = np.asarray(a, np.float64) - b
    den = float(np.linalg.norm(b))
    n = float(np.linalg.norm(d))
    return n / den if den > 0 else n
