"""Parity of the FP8 ReLU^2 MLP (through the C interface) with the CPU oracle.

Stage-wise, each GPU stage against the oracle's stage fed the GPU's own
inputs to it, with the bars of the QKV path:
  * e4m3 codes and scales (W1, W2 in both layouts, x8, h8, dy8, dpre8) and
    the zero token rows of the FP8 copies: bit-exact;
  * the bf16 outputs of GEMMs (h = relu(pre)^2, y, dpre, dX): per row, the
    distance to the exact float64 result may exceed what rounding that
    result to bf16 costs by at most 1.1x + 1e-3;
  * dW1, dW2 (fp32): <= 1e-3 relative per row.
End to end from x, W1, W2 and dy alone: y, dX, dW1 and dW2 no further
from the unquantised float64 results, in their worst row, than 1.1x the
oracle's own worst row + 1e-3.  (A one-ulp bf16 difference in h can move
an h8 code by one e4m3 step, 12.5%, so y is not compared with the
oracle's chain row by row.)
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_packed_reduced_amd import inputs

from gpu_run import bf16_gemm_excess, bf16_to_f64, row_rel_err, run_mlp, say

pytestmark = pytest.mark.gpu

GEMM_TOL = 1e-3

# K tails in every GEMM (D = 192 and F = 320 are not multiples of 128) and a
# ragged last token tile
MLP_TAILS = dict(n_seq=1, seq_len=333, d_model=192, d_ff=320)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build(force=False)


def _check_bf16_gemm(name, gpu_bits, exact):
    worst, excess = bf16_gemm_excess(gpu_bits, exact, oracle.round_bf16)
    say(f"[gpu] {name}: worst e_gpu - e_round {worst:.2e}, vs bar {excess:.2e}")
    assert excess <= GEMM_TOL, name


def _check_stages(w, r, fmt="e4m3"):
    T, D, F = r["T"], w["d_model"], w["d_ff"]
    wq = oracle.mlp_quantize_weights(r["w1"], r["w2"])
    for k in ("w1", "w1_t", "w2", "w2_t"):
        assert np.array_equal(r["c_" + k], wq[k.replace("_", "")]), k
    assert np.array_equal(r["w_scales"],
                          np.array([wq["s_w1"], wq["inv_w1"], wq["s_w2"], wq["inv_w2"]],
                                   np.float32))
    # forward: x8 exact; h against the exact relu(pre)^2 of the GPU's x8
    fw = oracle.mlp_forward(r["x_bits"], wq)
    assert np.array_equal(r["x8"], fw["x8"])
    assert r["x_scales"][0] == fw["s_x"] and r["x_scales"][1] == fw["inv_x"]
    assert not r["x8_tail"].any()
    _check_bf16_gemm("h", r["h"], fw["h64"])
    # h8 from the GPU's h: exact; y against the exact product of the GPU's h8
    fw2 = oracle.mlp_forward(r["x_bits"], wq, h_bits=r["h"])
    assert np.array_equal(r["h8"], fw2["h8"])
    assert r["h_scales"][0] == fw2["s_h"] and r["h_scales"][1] == fw2["inv_h"]
    assert not r["h8_tail"].any()
    _check_bf16_gemm("y", r["y"], fw2["y64"])
    # backward from the GPU's saved x8, h8
    s_x, s_h = np.float32(r["x_scales"][0]), np.float32(r["h_scales"][0])
    bw = oracle.mlp_backward(r["dy"], r["x8"], s_x, r["h8"], s_h, wq, grad_fmt=fmt)
    assert np.array_equal(r["dy8"], bw["dy8"])
    assert r["dy_scales"][0] == bw["s_dy"] and r["dy_scales"][1] == bw["inv_dy"]
    _check_bf16_gemm("dpre", r["dpre"], bw["dpre64"])
    bw2 = oracle.mlp_backward(r["dy"], r["x8"], s_x, r["h8"], s_h, wq, dpre_bits=r["dpre"],
                              grad_fmt=fmt)
    assert np.array_equal(r["dp8"], bw2["dp8"])
    assert r["dp_scales"][0] == bw2["s_dp"] and r["dp_scales"][1] == bw2["inv_dp"]
    assert not r["dp8_tail"].any()
    _check_bf16_gemm("dx", r["dx"], bw2["dx64"])
    e1 = row_rel_err(r["dw1"], bw2["dw1_64"])
    e2 = row_rel_err(r["dw2"], bw2["dw2_64"])
    say(f"[gpu] dw1 {e1:.2e} dw2 {e2:.2e}")
    assert e1 <= GEMM_TOL and e2 <= GEMM_TOL
    assert r["status"] == 0


@pytest.mark.parametrize("name,w", [("tiny", inputs.MLP_WORKLOADS["mlp_tiny"]),
                                    ("tails", MLP_TAILS),
                                    ("one_token", dict(n_seq=1, seq_len=1, d_model=128, d_ff=128)),
                                    ("block_plus_one",
                                     dict(n_seq=1, seq_len=257, d_model=64, d_ff=64))])
def test_mlp_stagewise(name, w):
    _check_stages(w, run_mlp(w, seed=42))


@pytest.mark.parametrize("name,w", [("tiny", inputs.MLP_WORKLOADS["mlp_tiny"]),
                                    ("tails", MLP_TAILS)])
def test_mlp_e5m2_gradients_stagewise(name, w):
    """dy8 and dpre8 in e5m2: codes and scales bit-exact, the GEMMs that read
    them (dh, dX, dW1, dW2: e5m2 x e4m3 on the matrix cores) to the bars."""
    _check_stages(w, run_mlp(w, seed=42, grad_format=1), fmt="e5m2")


def test_mlp_end_to_end_against_oracle_chain():
    w = inputs.MLP_WORKLOADS["mlp_tiny"]
    r = run_mlp(w, seed=7)
    wq = oracle.mlp_quantize_weights(r["w1"], r["w2"])
    fw = oracle.mlp_forward(r["x_bits"], wq)
    bw = oracle.mlp_backward(r["dy"], fw["x8"], fw["s_x"], fw["h8"], fw["s_h"], wq)
    # unquantised float64 gradients
    x = bf16_to_f64(r["x_bits"])
    w1, w2 = r["w1"].astype(np.float64), r["w2"].astype(np.float64)
    dy = bf16_to_f64(r["dy"])
    pre = x @ w1
    h = np.maximum(pre, 0.0) ** 2
    dpre = 2.0 * (dy @ w2.T) * np.maximum(pre, 0.0)
    ref = dict(y=h @ w2, dx=dpre @ w1.T, dw1=x.T @ dpre, dw2=h.T @ dy)
    gpu = dict(y=bf16_to_f64(r["y"]), dx=bf16_to_f64(r["dx"]), dw1=r["dw1"], dw2=r["dw2"])
    orc = dict(y=bf16_to_f64(fw["y_bits"]), dx=bf16_to_f64(bw["dx_bits"]), dw1=bw["dw1_64"],
               dw2=bw["dw2_64"])
    # worst row of each (token rows of y and dX, rows of dW1 [D][F] and
    # dW2 [F][D])
    for k in ref:
        eg, eo = row_rel_err(gpu[k], ref[k]), row_rel_err(orc[k], ref[k])
        say(f"[gpu] mlp e2e {k}: worst row gpu {eg:.3e} oracle {eo:.3e}")
        assert eg <= 1.1 * eo + 1e-3, k


def test_mlp_deterministic_and_zero_input():
    w = MLP_TAILS
    a = run_mlp(w, seed=5)
    b = run_mlp(w, seed=5)
    for k in ("h", "h8", "y", "dpre", "dp8", "dx", "dw1", "dw2"):
        assert np.array_equal(a[k], b[k]), k
    T = w["n_seq"] * w["seq_len"]
    z = run_mlp(w, seed=5, x_bits=np.zeros((T, w["d_model"]), np.uint16))
    for k in ("h", "y", "dpre", "dx"):  # values (a product of zeros may be -0)
        assert not (bf16_to_f64(z[k]) != 0).any(), k
    assert not (z["dw1"] != 0).any() and not (z["dw2"] != 0).any()
    assert z["h_scales"][0] == 1.0 and z["status"] == 0


def test_mlp_nonfinite_input_sets_status():
    w = MLP_TAILS
    T = w["n_seq"] * w["seq_len"]
    x = inputs.make_x(w, 3)
    x[5, 7] = 0x7FC0
    r = run_mlp(w, seed=3, x_bits=x, backward=False)
    assert r["status"] & 2


@pytest.mark.parametrize("name,w", [("tiny", inputs.MLP_WORKLOADS["mlp_tiny"]),
                                    ("tails", MLP_TAILS),
                                    ("one_token", dict(n_seq=1, seq_len=1, d_model=128, d_ff=128)),
                                    ("mlp_64k", inputs.MLP_WORKLOADS["mlp_64k"])])
def test_mlp_pack_forward_matches_separate_calls(name, w):
    """mlp_pack_forward (the weight pack and the forward with their
    quantiser launches shared) writes what mlp_pack_quantize_weights and
    mlp_forward write, bit for bit: both layouts of W1 and W2 and their
    scales, x8 and h8 with their zero tails and scales, y; the backward
    from its cache and saved buffer then matches; and it clears the status
    word it was handed with every bit set."""
    sep = run_mlp(w, seed=29)
    one = run_mlp(w, seed=29, pack_forward=True)
    for k in ("c_w1", "c_w1_t", "c_w2", "c_w2_t", "w_scales", "x8", "x8_tail", "h8", "h8_tail",
              "x_scales", "h_scales", "y", "dp8", "dx"):
        assert np.array_equal(sep[k], one[k]), k
    for k in ("dw1", "dw2"):
        assert np.array_equal(sep[k].view(np.uint32), one[k].view(np.uint32)), k
    assert sep["status"] == one["status"] == 0


def test_mlp_pack_forward_status_bits():
    """NaNs in W2 and in x set the weight and the activation bits in the
    combined call as in the separate calls."""
    w = MLP_TAILS
    x = inputs.make_x(w, 6)
    x[3, 1] = 0x7FC0
    w1, w2 = inputs.make_mlp_w(w, 7)
    w2[2, 5] = np.nan
    sep = run_mlp(w, seed=6, x_bits=x, w12=(w1, w2), backward=False)
    one = run_mlp(w, seed=6, x_bits=x, w12=(w1, w2), backward=False, pack_forward=True)
    assert sep["status"] & 3 == 3
    assert sep["status"] == one["status"]


def test_mlp_64k_sampled():
    """The benchmark's MLP workload (T = 65536, D = 768, d_ff = 3072) in its
    launch configuration: every e4m3 code of x8, h8, dy8 and dpre8 bit-exact
    against the oracle's quantiser of the GPU's own input to it; sampled
    token rows of h, y, dpre and dX, and sampled rows of dW1 and dW2, against
    the oracle computed row by row."""
    w = inputs.MLP_WORKLOADS["mlp_64k"]
    r = run_mlp(w, seed=42)
    T, D, F = r["T"], w["d_model"], w["d_ff"]
    wq = oracle.mlp_quantize_weights(r["w1"], r["w2"])
    for k in ("w1", "w1_t", "w2", "w2_t"):
        assert np.array_equal(r["c_" + k], wq[k.replace("_", "")]), k
    x8, s_x, _, _ = oracle.quantize_bf16(r["x_bits"])
    assert np.array_equal(r["x8"], x8) and r["x_scales"][0] == s_x
    h8, s_h, _, _ = oracle.quantize_bf16(r["h"])
    assert np.array_equal(r["h8"], h8) and r["h_scales"][0] == s_h
    dy8, s_dy, _, _ = oracle.quantize_bf16(r["dy"])
    assert np.array_equal(r["dy8"], dy8) and r["dy_scales"][0] == s_dy
    dp8, s_dp, _, _ = oracle.quantize_bf16(r["dpre"])
    assert np.array_equal(r["dp8"], dp8) and r["dp_scales"][0] == s_dp
    assert not r["x8_tail"].any() and not r["h8_tail"].any() and not r["dp8_tail"].any()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 1, T // 2, T - 2, T - 1], rng.integers(0, T, 27)]))
    say(f"[gpu] mlp 64k: checking {rows.size} token rows")
    w1c = wq["w1"]
    h_exact = oracle.relu2(oracle.gemm_e4m3(x8[rows], w1c, s_x, wq["s_w1"]))
    _check_bf16_gemm("h rows", r["h"][rows], h_exact)
    _check_bf16_gemm("y rows", r["y"][rows], oracle.gemm_e4m3(h8[rows], wq["w2"], s_h, wq["s_w2"]))
    dh = oracle.gemm_e4m3(dy8[rows], np.ascontiguousarray(wq["w2"].T), s_dy, wq["s_w2"])
    dpre_exact = oracle.relu2_grad(dh, float(s_h) * oracle.e4m3_decode(h8[rows]))
    _check_bf16_gemm("dpre rows", r["dpre"][rows], dpre_exact)
    _check_bf16_gemm("dx rows", r["dx"][rows],
                     oracle.gemm_e4m3(dp8[rows], np.ascontiguousarray(w1c.T), s_dp, wq["s_w1"]))
    # dW1 rows i: x8[:, i]^T dpre8; dW2 rows f: h8[:, f]^T dy8
    tab = oracle.e4m3_decode_table()
    di, df = [0, 383, D - 1], [0, 1537, F - 1]
    w1_rows, w2_rows = np.zeros((len(di), F)), np.zeros((len(df), D))
    for t0 in range(0, T, 8192):  # float64 sums over token chunks
        sl = slice(t0, t0 + 8192)
        w1_rows += tab[x8[sl][:, di]].T @ tab[dp8[sl]]
        w2_rows += tab[h8[sl][:, df]].T @ tab[dy8[sl]]
    e1 = row_rel_err(r["dw1"][di], float(s_x) * float(s_dp) * w1_rows)
    e2 = row_rel_err(r["dw2"][df], float(s_h) * float(s_dy) * w2_rows)
    say(f"[gpu] mlp 64k dw1 rows {e1:.2e} dw2 rows {e2:.2e}")
    assert e1 <= GEMM_TOL and e2 <= GEMM_TOL
    assert r["status"] == 0
