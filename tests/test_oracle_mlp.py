"""Pins of the oracle's FP8 ReLU^2 MLP (PR #344 page, "Changes": the FP8
MLP forward and backward, relu(pre) rebuilt from the stored squared
activation).

* ``relu2_grad`` against central differences of ``relu2``;
* a structured case in which every e4m3 quantisation and every rounding is
  exact, so each output of ``mlp_forward`` / ``mlp_backward`` must equal the
  value worked out from the construction in plain integer arithmetic here:
  each column of W1 and W2 holds one nonzero, so every y, dh, dpre and dx
  entry is a single product and a transposed operand, a wrong index, a lost
  factor 2 or a missing square root changes it;
* the FP8 chain on the seeded tiny workload against the float64 gradient
  that torch's autograd takes of the unquantised MLP, within FP8 noise.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_packed_reduced_amd import inputs


def test_relu2_grad_matches_central_differences():
    rng = np.random.default_rng(3)
    pre = rng.standard_normal(4000)
    pre = pre[np.abs(pre) > 1e-3]          # away from the kink
    dh = rng.standard_normal(pre.size)
    eps = 1e-6
    fd = (oracle.relu2(pre + eps) - oracle.relu2(pre - eps)) / (2 * eps)
    got = oracle.relu2_grad(dh, oracle.relu2(pre))
    assert np.allclose(got, dh * fd, rtol=1e-6, atol=1e-9)
    # negative pre: zero activation, zero gradient
    neg = pre < 0
    assert not oracle.relu2(pre[neg]).any() and not got[neg].any()


# ------------------------------------------------ exact structured case

T, D, F = 6, 32, 24
NF = 20            # columns 0 .. NF-1 of W1 / rows of W2 carry the signal
F_ZERO = 20        # a row of h that is zero for every token
X_BIG, W1_BIG = 30, 31   # x column holding 448; W1 row holding 448
D_BIG = 31         # dy / W2 column holding the large entries


def _bf16_bits(v: float) -> int:
    """bf16 pattern of a value that is exactly representable."""
    b = np.array([v], dtype=np.float32).view(np.uint32)[0]
    assert b & 0xFFFF == 0, v
    return int(b >> 16)


def _structured():
    rng = np.random.default_rng(11)
    perm_i = rng.permutation(NF)           # W1 column f reads x column i(f) = perm_i[f]
    sig1 = rng.choice([-1, 1], NF)
    perm_f = rng.permutation(NF)           # W2 column d (< NF) reads h column f(d)
    sig2 = rng.choice([-1, 1], NF)
    w1 = np.zeros((D, F), np.float32)
    for f in range(NF):
        w1[perm_i[f], f] = 7 * sig1[f]
    w1[W1_BIG, F_ZERO + 1] = 448           # x column W1_BIG is zero: no effect
    w2 = np.zeros((F, D), np.float32)
    for d in range(NF):
        w2[perm_f[d], d] = sig2[d]
    w2[F_ZERO, D_BIG] = 448                # h column F_ZERO is zero
    x = np.zeros((T, D), np.float32)
    x[:, :NF] = rng.choice([0, 1, -1, 2, -2, 4, -4, 8, -8], (T, NF))
    x[1, perm_i[0]] = 8 * sig1[0]          # pre = 56 somewhere: amax(h) = 3136
    x[0, X_BIG] = 448                      # W1 row X_BIG is zero
    dy = np.zeros((T, D), np.float32)
    dy[:, :NF] = rng.choice([0, 1, -1], (T, NF)) * 2.0 ** rng.integers(-6, -1, (T, NF))
    dy[2, D_BIG] = 56                      # amax(dy) = 56: s_dy = 1/8 exactly
    return x, w1, w2, dy, perm_i, sig1, perm_f, sig2


def _expected(x, w1, w2, dy, perm_i, sig1, perm_f, sig2):
    """Every output from the construction, in integers / dyadic rationals."""
    xi = x.astype(np.int64)
    pre = np.zeros((T, F), np.int64)
    for t in range(T):
        for f in range(NF):
            pre[t, f] = 7 * sig1[f] * xi[t, perm_i[f]]
    h = np.maximum(pre, 0) ** 2
    y = np.zeros((T, D), np.float64)
    for t in range(T):
        for d in range(NF):
            y[t, d] = sig2[d] * h[t, perm_f[d]]
    inv_f = {int(perm_f[d]): d for d in range(NF)}
    dh = np.zeros((T, F), np.float64)
    for t in range(T):
        for f in range(NF):
            if f in inv_f:
                dh[t, f] = sig2[inv_f[f]] * float(dy[t, inv_f[f]])
        dh[t, F_ZERO] = 448.0 * float(dy[t, D_BIG])
    dpre = 2.0 * dh * np.sqrt(h)
    dx = np.zeros((T, D), np.float64)
    for t in range(T):
        for f in range(NF):
            dx[t, perm_i[f]] = dpre[t, f] * 7 * sig1[f]
    dw1 = np.zeros((D, F), np.float64)
    dw2 = np.zeros((F, D), np.float64)
    for i in range(D):
        for f in range(F):
            dw1[i, f] = sum(float(x[t, i]) * dpre[t, f] for t in range(T))
    for f in range(F):
        for d in range(D):
            dw2[f, d] = sum(float(h[t, f]) * float(dy[t, d]) for t in range(T))
    return dict(h=h, y=y, dpre=dpre, dx=dx, dw1=dw1, dw2=dw2)


@pytest.mark.parametrize("fmt,s_dy", [("e4m3", 0.125), ("e5m2", 2.0 ** -10)])
def test_structured_mlp_is_exact(fmt, s_dy):
    """Both gradient formats: dy's scale is a power of two in each (56/448,
    56/57344), and every dy and dpre value is exact in both."""
    x, w1, w2, dy, *perm = _structured()
    e = _expected(x, w1, w2, dy, *perm)
    wq = oracle.mlp_quantize_weights(w1, w2)
    assert wq["s_w1"] == 1 and wq["s_w2"] == 1 and wq["rc"] == 0
    x_bits = np.vectorize(_bf16_bits)(x).astype(np.uint16)
    fw = oracle.mlp_forward(x_bits, wq)
    assert fw["s_x"] == 1 and fw["s_h"] == 7
    assert np.array_equal(oracle.bf16_to_f64(fw["h_bits"]), e["h"])
    assert np.array_equal(float(fw["s_h"]) * oracle.e4m3_decode(fw["h8"]), e["h"])
    assert np.array_equal(oracle.bf16_to_f64(fw["y_bits"]), e["y"])
    dy_bits = np.vectorize(_bf16_bits)(dy).astype(np.uint16)
    bw = oracle.mlp_backward(dy_bits, fw["x8"], fw["s_x"], fw["h8"], fw["s_h"], wq, grad_fmt=fmt)
    assert bw["s_dy"] == s_dy
    dec = oracle.e5m2_decode if fmt == "e5m2" else oracle.e4m3_decode
    assert np.array_equal(float(bw["s_dy"]) * dec(bw["dy8"]), dy.astype(np.float64))
    assert np.array_equal(oracle.bf16_to_f64(bw["dpre_bits"]), e["dpre"])
    # dpre's scale is a power of two, so its codes are exact too
    assert np.array_equal(float(bw["s_dp"]) * dec(bw["dp8"]), e["dpre"])
    assert np.array_equal(oracle.bf16_to_f64(bw["dx_bits"]), e["dx"])
    assert np.array_equal(bw["dw1_f32"].astype(np.float64), e["dw1"])
    assert np.array_equal(bw["dw2_f32"].astype(np.float64), e["dw2"])
    # the case is not degenerate
    assert np.count_nonzero(e["dpre"]) > 20 and np.count_nonzero(e["dw1"]) > 20


# ----------------------------------- FP8 chain vs unquantised autograd

def test_fp8_chain_tracks_float64_autograd():
    w = inputs.MLP_WORKLOADS["mlp_tiny"]
    x_bits = inputs.make_x(w, 42)
    w1, w2 = inputs.make_mlp_w(w, 43)
    dy_bits = inputs.make_mlp_dy(w, 44)
    wq = oracle.mlp_quantize_weights(w1, w2)
    fw = oracle.mlp_forward(x_bits, wq)
    bw = oracle.mlp_backward(dy_bits, fw["x8"], fw["s_x"], fw["h8"], fw["s_h"], wq)
    xt = torch.tensor(oracle.bf16_to_f64(x_bits), requires_grad=True)
    w1t = torch.tensor(w1.astype(np.float64), requires_grad=True)
    w2t = torch.tensor(w2.astype(np.float64), requires_grad=True)
    y = torch.relu(xt @ w1t).square() @ w2t
    y.backward(torch.tensor(oracle.bf16_to_f64(dy_bits)))

    def rel(got, want):
        want = np.asarray(want)
        return float(np.linalg.norm(got - want) / np.linalg.norm(want))

    errs = dict(y=rel(oracle.bf16_to_f64(fw["y_bits"]), y.detach().numpy()),
                dx=rel(oracle.bf16_to_f64(bw["dx_bits"]), xt.grad.numpy()),
                dw1=rel(bw["dw1_64"], w1t.grad.numpy()),
                dw2=rel(bw["dw2_64"], w2t.grad.numpy()))
    print(errs)
    # e4m3 keeps 3 fraction bits (rounding error up to 2^-4); each output
    # here passes through two to five quantised tensors
    for k, e in errs.items():
        assert e < 0.12, (k, e)
