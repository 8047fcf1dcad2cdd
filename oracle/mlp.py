"""MLP form of the chain, O = act(X.W1).W2, and its gated form -- oracle (test
infrastructure).

Source: METP abstract (the chain O = f(A.B).C with an optional function between
the two products) and TSP article, "Lo que realmente significa plegar" (the MLP
weights are split into shards whose partial outputs are summed locally).  The
pages never name the activation; GeLU is taken in its exact form
x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) (Hendrycks and Gimpel, "Gaussian Error
Linear Units"), with that paper's tanh approximation and the identity as
options.  Float64, no intermediate rounding.

Gated form: the TSP article ("Lo que realmente significa plegar") runs a gated
MLP whose shards are gate, up and down projections.  Reading, as the plainest
form of such a layer: O = (act(X.Wg) * (X.Wu)).Wd with * elementwise; the
activation is applied to the gate product only.  The page does not name the
activation either; SiLU, z * sigmoid(z), is the default here, with the GeLU
forms and the identity as options.
"""

import math

import numpy as np
from scipy.special import erf, expit


def gelu_erf(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def gelu_tanh(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def silu(z):
    """z * sigmoid(z) (sigmoid by scipy's overflow-safe expit)."""
    z = np.asarray(z, dtype=np.float64)
    return z * expit(z)


def _identity(z):
    return np.asarray(z, dtype=np.float64)


ACTIVATIONS = {"gelu_erf": gelu_erf, "gelu_tanh": gelu_tanh, "identity": _identity, "silu": silu}


def mlp(x, w1, w2, act="gelu_erf"):
    """x [M, K], w1 [K, N], w2 [N, K2] -> O [M, K2] float64."""
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    if x.shape[1] != w1.shape[0] or w1.shape[1] != w2.shape[0]:
        raise ValueError(f"shape mismatch X{x.shape} W1{w1.shape} W2{w2.shape}")
    h = ACTIVATIONS[act](x @ w1)
    return h @ w2


def mlp_gated(x, wg, wu, wd, act="silu"):
    """x [M, K], wg and wu [K, N], wd [N, K2] -> O = (act(x.wg) * (x.wu)).wd, float64."""
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(wg, dtype=np.float64)
    wu = np.asarray(wu, dtype=np.float64)
    wd = np.asarray(wd, dtype=np.float64)
    if wg.shape != wu.shape or x.shape[1] != wg.shape[0] or wg.shape[1] != wd.shape[0]:
        raise ValueError(f"shape mismatch X{x.shape} Wg{wg.shape} Wu{wu.shape} Wd{wd.shape}")
    h = ACTIVATIONS[act](x @ wg) * (x @ wu)
    return h @ wd
