"""Pure-Python brute force of the fused SwiGLU MLP for tiny shapes (test
infrastructure only; no NumPy, no C).

It exists to check the C oracle's indexing on shapes small enough to write
out by hand: out = silu(x.Wgate) * (x.Wup), y = out.Wdown, following the
problem statement of "Tile-Level Activation Overlap for Efficient LLM
Inference" and the projection table of "Anatomie d'un transformeur sur GPU"
§1.2.  Inputs are nested lists of Python floats (fp64).
"""
import math


def sigmoid(z):
    # 1 / (1 + e^-z), using e^z / (1 + e^z) for negative z to avoid overflow
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    e = math.exp(z)
    return e / (1.0 + e)


def swiglu(x, wg, wu):
    M, d, dff = len(x), len(wg), len(wg[0])
    out = [[0.0] * dff for _ in range(M)]
    for m in range(M):
        for n in range(dff):
            g = 0.0
            u = 0.0
            for k in range(d):
                g += x[m][k] * wg[k][n]
                u += x[m][k] * wu[k][n]
            out[m][n] = g * sigmoid(g) * u
    return out


def mlp(x, wg, wu, wd):
    h = swiglu(x, wg, wu)
    M, dff, d = len(h), len(wd), len(wd[0])
    y = [[0.0] * d for _ in range(M)]
    for m in range(M):
        for j in range(d):
            s = 0.0
            for n in range(dff):
                s += h[m][n] * wd[n][j]
            y[m][j] = s
    return y
