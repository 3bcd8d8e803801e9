"""Parity of the HIP path (through the C interface) with the CPU oracle.

Stage-wise: every GPU stage is compared with the oracle's stage fed the
GPU's own inputs to that stage.  Bars:
  * FP8 codes and scales, the zero token rows padding the FP8 copies to a
    whole K step, the V relayout: bit-exact;
  * GEMM outputs: the accumulated product must be within 1e-3 per row norm.
    dW is fp32 and is compared directly: ||gpu - oracle|| / ||oracle|| <= 1e-3
    per row.  The projection Y and dX are rounded to bf16, whose own rounding
    costs ~2e-3 per row, so per row their distance to the exact float64
    product may exceed what rounding the exact product costs by at most
    1.1x + 1e-3 (the protocol the end-to-end check uses too).  The matrix
    cores' FP8 dot products carry ~14-15 significant bits in their partial
    sums, which flips a few bf16 roundings; compared directly with the
    bf16-rounded oracle the worst row of a K=128 product reaches ~1.2e-3;
  * normalised / rotated q, k and the packed gradient dQKV: <= 1e-2 per
    (token, head) row.  For head widths 64, 96 and 128 the norm and RoPE run
    in the forward GEMM's epilogue and its pre-norm rows never reach memory:
    the oracle's norm/RoPE stage is then fed the oracle's own bf16 product of
    the GPU's FP8 codes (the codes are bit-exact, so this is the same
    product up to accumulation order), and the GEMM bar applies to the V
    columns.  The saved 1/rms of every Q/K head row follows the GEMM
    protocol: per row, its relative distance to the 1/rms of the exact
    float64 product may exceed what rounding that product to bf16 moves the
    row by at most 1.1x + 1e-3 (1/rms scales with 1 / ||row||, so it moves
    by no more than the row).  Other widths keep the pre-norm rows (in the
    forward workspace) and are checked on them;
End to end (from x, W and the upstream gradients alone): q, k, v <= 1e-2;
dX and dW, whose FP8 gradient codes can flip where the bf16 dQKV differs
by one ulp, must be no further from the unquantised float64 result than
1.1 x the oracle's own distance + 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_packed_reduced_amd import inputs

from gpu_run import (BASE, EPS, bf16_gemm_excess, bf16_to_f64, rho_rows, row_errors,
                     row_rel_err, run, say)

pytestmark = pytest.mark.gpu

GEMM_TOL = 1e-3
NORM_TOL = 1e-2

RAGGED = dict(n_seq=3, seq_len=100, d_model=128, n_heads=2, d_qk=96, d_v=128)
SMALL_16K_DIMS = dict(n_seq=2, seq_len=384, d_model=768, n_heads=6, d_qk=96, d_v=128)
# K tails in both bf16-output GEMMs (d_model 192 and N = 320 are not multiples
# of 128) and a head width outside the quad-lane norm/RoPE kernels (48)
TAILS = dict(n_seq=2, seq_len=77, d_model=192, n_heads=2, d_qk=48, d_v=64)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build(force=False)


def _dims(w):
    return inputs.dims_of(w)


# ------------------------------------------------------------------ encoder

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encoder_matches_oracle_on_every_rounding_class(fmt):
    from fp8_packed_reduced_amd import binding as B
    e5 = fmt == "e5m2"
    enc = oracle.e5m2_encode if e5 else oracle.e4m3_encode
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    tails = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    v = (hi[:, None] | tails[None, :]).ravel().view(np.float32)
    v = v[np.isfinite(v)]
    v = v[: (v.size // 16) * 16]
    say(f"[gpu] {fmt} encoder sweep over {v.size} fp32 patterns")
    got = B.e4m3_encode(torch.from_numpy(v).cuda(), 1.0, e5m2=e5).cpu().numpy()
    assert np.array_equal(got, enc(v))
    # with a scale: codes of fl32(v * inv)
    rng = np.random.default_rng(1)
    r = rng.standard_normal(1 << 20).astype(np.float32)
    inv = np.float32(57344.0 if e5 else 448.0) / np.float32(np.abs(r).max())
    got = B.e4m3_encode(torch.from_numpy(r).cuda(), float(inv), e5m2=e5).cpu().numpy()
    assert np.array_equal(got, enc(r * inv))


# ------------------------------------------------------------ weight quant

@pytest.mark.parametrize("wl", ["tiny", "fwd_16k", "sweep_64", "sweep_128"])
def test_pack_quantize_bit_exact(wl):
    w = dict(inputs.WORKLOADS[wl], n_seq=1, seq_len=128)
    r = run(w, seed=5, backward=False)
    wp, wpt, s, inv, rc = oracle.pack_quantize_weights(_dims(w), r["W"])
    assert np.array_equal(r["w_packed"], wp)
    assert np.array_equal(r["w_packed_t"], wpt)
    assert r["w_scales"][0] == s and r["w_scales"][1] == inv
    assert r["status"] == 0


def test_pack_flags_nonfinite_weights():
    w = dict(inputs.WORKLOADS["tiny"], seq_len=128)
    W = inputs.make_w(w, 3)
    W[5, 7] = np.inf
    r = run(w, seed=3, W=W, backward=False)
    assert r["status"] & 1


# ------------------------------------------------------------ forward

def _prenorm_bits(w, r, rows=None):
    """The bf16 pre-norm Q|K rows the GPU's norm/RoPE stage worked on: its own
    (where they are stored), else the oracle's product of the GPU's codes
    (the codes are bit-exact against the oracle's quantisers)."""
    nqk2 = 2 * w["n_heads"] * w["d_qk"]
    if r["qk_pre"] is not None:
        return r["qk_pre"] if rows is None else r["qk_pre"][rows]
    x8 = r["x8"] if rows is None else r["x8"][rows]
    return oracle.round_bf16(oracle.gemm_e4m3(x8, r["w_packed"][:, :nqk2], r["x_scales"][0],
                                              r["w_scales"][0]))


def _rho_excess(rho_gpu, y64_qk, H, dqk):
    """Worst row of |rho_gpu / rho_exact - 1| - 1.1 e_round, rho_exact the
    oracle's 1/rms of the exact product's head row and e_round the relative
    distance that rounding that row to bf16 moves it (rho_gpu: [T][2H])."""
    y = y64_qk.reshape(y64_qk.shape[0], 2 * H, dqk)
    rho_exact = oracle.rmsnorm(y, EPS)[1][..., 0]
    e_round = row_errors(bf16_to_f64(oracle.round_bf16(y)), y).reshape(rho_exact.shape)
    e_gpu = np.abs(rho_gpu / rho_exact - 1.0)
    return float(np.max(e_gpu - 1.1 * e_round)), float(np.max(e_gpu))


def _check_forward(w, r):
    dims = _dims(w)
    n_seq, S = w["n_seq"], w["seq_len"]
    T, H, dqk, dv = r["T"], w["n_heads"], w["d_qk"], w["d_v"]
    nqk2 = 2 * H * dqk
    # a2: activation quantiser, bit-exact; padding columns and the token
    # rows up to the padded count (the dW GEMM's K tail) zero
    x8, s_x, inv_x, _ = oracle.quantize_bf16(r["x_bits"])
    assert np.array_equal(r["x8"], x8) and not r["x8_kpad"].any()
    assert r["x_scales"][0] == s_x and r["x_scales"][1] == inv_x
    assert not r["x8_tail"].any()
    # a3: packed GEMM from the GPU's own codes: the V columns (and the
    # stored pre-norm rows where there are any)
    y = oracle.gemm_e4m3(r["x8"], r["w_packed"], r["x_scales"][0], r["w_scales"][0])
    gpu_v = oracle.from_head_major(r["v"]).reshape(T, H * dv)
    x_gemm, over_gemm = bf16_gemm_excess(gpu_v, y[:, nqk2:], oracle.round_bf16)
    if r["qk_pre"] is not None:
        x_qk, over_qk = bf16_gemm_excess(r["qk_pre"], y[:, :nqk2], oracle.round_bf16)
        x_gemm, over_gemm = max(x_gemm, x_qk), max(over_gemm, over_qk)
    # a4: norm/RoPE fed the pre-norm rows (the GPU's, else the oracle's
    # product of the GPU's codes)
    a_bits = _prenorm_bits(w, r)
    y_bits = oracle.round_bf16(y)
    y_bits[:, :nqk2] = a_bits
    o = oracle.qkv_forward(dims, n_seq, S, r["x_bits"], r["w_packed"], r["w_scales"][0],
                           y_bits=y_bits)
    e_q = row_rel_err(bf16_to_f64(r["q"]), o["q64"])
    e_k = row_rel_err(bf16_to_f64(r["k"]), o["k64"])
    over_rho, e_rho = _rho_excess(rho_rows(r["rho"]), y[:, :nqk2], H, dqk)
    say(f"[gpu] forward errors ({'fused' if r['fused'] else 'unfused'}): gemm excess over bf16 "
        f"rounding {x_gemm:.2e} q {e_q:.2e} k {e_k:.2e} rho {e_rho:.2e} (excess {over_rho:.2e})")
    assert over_gemm <= GEMM_TOL and over_rho <= GEMM_TOL
    assert e_q <= NORM_TOL and e_k <= NORM_TOL


def _check_backward(w, r, fmt="e4m3"):
    dims = _dims(w)
    n_seq, S = w["n_seq"], w["seq_len"]
    T, H, dqk = r["T"], w["n_heads"], w["d_qk"]
    nqk2 = 2 * H * dqk
    dq, dk, dv = r["dy"]
    # a5: norm/RoPE backward; the oracle's backward runs on the pre-norm rows
    # (its definition), the GPU's on its q, k and saved 1/rms
    ob = oracle.qkv_backward(dims, n_seq, S, dq, dk, dv, r["x8"], r["x_scales"][0],
                             _prenorm_bits(w, r), r["w_packed"], r["w_scales"][0], grad_fmt=fmt)
    g = r["dqkv"]
    e_dqk = row_rel_err(bf16_to_f64(g[:, :nqk2]).reshape(T, 2 * H, dqk),
                        ob["dqkv64"][:, :nqk2].reshape(T, 2 * H, dqk))
    # the packed V part is dv itself, which the gradient quantiser reads
    # head-major: its codes below are what checks that read
    assert np.array_equal(g[:, nqk2:], ob["dqkv_bits"][:, nqk2:])
    # a6: gradient quantiser, bit-exact on the GPU's own dQKV
    g8, s_g, inv_g, _ = oracle.quantize_bf16(g, fmt)
    assert np.array_equal(r["g8"], g8) and not r["g8_kpad"].any()
    assert r["g_scales"][0] == s_g and r["g_scales"][1] == inv_g
    assert not r["g8_tail"].any()
    # a7, a8: GEMMs from the GPU's own codes
    dx64 = oracle.gemm_e4m3(r["g8"], np.ascontiguousarray(r["w_packed"].T), s_g, r["w_scales"][0],
                            a_fmt=fmt)
    e_dx = row_rel_err(bf16_to_f64(r["dx"]), bf16_to_f64(oracle.round_bf16(dx64)))
    x_dx, over_dx = bf16_gemm_excess(r["dx"], dx64, oracle.round_bf16)
    dw = oracle.round_f32(oracle.gemm_e4m3(np.ascontiguousarray(r["x8"].T), r["g8"],
                                           r["x_scales"][0], s_g, b_fmt=fmt))
    e_dw = row_rel_err(r["dw"], dw)
    say(f"[gpu] backward errors: dqkv {e_dqk:.2e} dx {e_dx:.2e} (excess {x_dx:.2e}) "
        f"dw {e_dw:.2e}")
    assert e_dqk <= NORM_TOL
    assert over_dx <= GEMM_TOL and e_dw <= GEMM_TOL


@pytest.mark.parametrize("name,w", [("tiny", inputs.WORKLOADS["tiny"]), ("ragged", RAGGED),
                                    ("d768", SMALL_16K_DIMS), ("tails", TAILS),
                                    ("one_token", dict(n_seq=1, seq_len=1, d_model=128,
                                                       n_heads=1, d_qk=96, d_v=128)),
                                    ("one_token_per_seq", dict(n_seq=5, seq_len=1, d_model=64,
                                                               n_heads=1, d_qk=96, d_v=128))])
def test_forward_backward_stagewise(name, w):
    r = run(w, seed=42)
    assert r["status"] == 0
    _check_forward(w, r)
    _check_backward(w, r)


@pytest.mark.parametrize("dqk", [64, 128])
def test_width_sweep_stagewise(dqk):
    w = dict(n_seq=1, seq_len=512, d_model=768, n_heads=6, d_qk=dqk, d_v=128)
    r = run(w, seed=7)
    _check_forward(w, r)
    _check_backward(w, r)


def test_forward_only_16k_shape_full():
    w = inputs.WORKLOADS["fwd_16k"]
    r = run(w, seed=42, backward=False)
    _check_forward(w, r)


# ---------------------------------------------------------- end to end

def _unquantised(w, x_bits, W, dy):
    """float64 result with no FP8 anywhere (reference for the e2e protocol)."""
    n_seq, S = w["n_seq"], w["seq_len"]
    T, H, dqk = n_seq * S, w["n_heads"], w["d_qk"]
    nq = H * dqk
    x = bf16_to_f64(x_bits)
    Wd = W.astype(np.float64)
    y = x @ Wd
    pos = oracle.positions_of(n_seq, S)
    dq, dk, dv = (bf16_to_f64(a) for a in dy)
    dqp = oracle.qk_norm_rope_bwd(y[:, :nq].reshape(T, H, dqk), oracle.from_head_major(dq), pos,
                                  EPS, BASE)
    dkp = oracle.qk_norm_rope_bwd(y[:, nq:2 * nq].reshape(T, H, dqk),
                                  oracle.from_head_major(dk), pos, EPS, BASE)
    g = np.concatenate([dqp.reshape(T, nq), dkp.reshape(T, nq),
                        oracle.from_head_major(dv).reshape(T, -1)], axis=1)
    return g @ Wd.T, x.T @ g


def test_end_to_end_against_oracle_chain():
    w = inputs.WORKLOADS["tiny"]
    dims = _dims(w)
    r = run(w, seed=42)
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, r["W"])
    of = oracle.qkv_forward(dims, 1, w["seq_len"], r["x_bits"], wp, s_w)
    e_q = row_rel_err(bf16_to_f64(r["q"]), of["q64"])
    e_k = row_rel_err(bf16_to_f64(r["k"]), of["k64"])
    e_v = row_rel_err(bf16_to_f64(r["v"]), of["v64"])
    assert max(e_q, e_k, e_v) <= NORM_TOL
    dq, dk, dv = r["dy"]
    ob = oracle.qkv_backward(dims, 1, w["seq_len"], dq, dk, dv, of["x8"], of["s_x"],
                             of["y_bits"][:, :2 * w["n_heads"] * w["d_qk"]], wp, s_w)
    dx_ref, dw_ref = _unquantised(w, r["x_bits"], r["W"], r["dy"])
    e_gpu_dx = row_rel_err(bf16_to_f64(r["dx"]), dx_ref)
    e_orc_dx = row_rel_err(bf16_to_f64(ob["dx_bits"]), dx_ref)
    e_gpu_dw = row_rel_err(r["dw"], dw_ref)
    e_orc_dw = row_rel_err(ob["dw_f32"], dw_ref)
    say(f"[gpu] e2e: q {e_q:.2e} k {e_k:.2e} v {e_v:.2e}; vs unquantised: dx gpu {e_gpu_dx:.3e} "
        f"oracle {e_orc_dx:.3e}; dw gpu {e_gpu_dw:.3e} oracle {e_orc_dw:.3e}")
    assert e_gpu_dx <= 1.1 * e_orc_dx + 1e-3
    assert e_gpu_dw <= 1.1 * e_orc_dw + 1e-3


# ------------------------------------------------------------ properties

def test_deterministic_rerun():
    w = RAGGED
    a = run(w, seed=9)
    b = run(w, seed=9)
    for key in ("q", "k", "v", "x8", "rho", "dqkv", "g8", "dx", "dw"):
        assert np.array_equal(a[key], b[key]), key


def test_scores_depend_only_on_position_difference():
    # every token has the same x row: pre-RoPE q and k are the same for all
    # positions, so q_m . k_n may only depend on m - n
    w = inputs.WORKLOADS["tiny"]
    row = inputs.make_x(dict(w, seq_len=1), 4)
    x_bits = np.repeat(row, w["seq_len"], axis=0)
    r = run(w, seed=4, x_bits=x_bits, backward=False)
    q = bf16_to_f64(r["q"][0, 0])
    k = bf16_to_f64(r["k"][0, 0])
    Sc = q @ k.T
    worst = max(np.ptp(np.diagonal(Sc, off)) for off in range(-255, 256))
    say(f"[gpu] max spread along a diagonal: {worst:.3e} (scores up to {np.abs(Sc).max():.1f})")
    assert worst <= 0.02 * np.abs(Sc).max()


@pytest.mark.parametrize("name,w,stride", [("tiny", inputs.WORKLOADS["tiny"], 128),
                                           ("ragged", RAGGED, 104), ("tails", TAILS, 64),
                                           ("d64", dict(RAGGED, d_qk=64), 128),
                                           ("d128", dict(RAGGED, d_qk=128), 136)])
def test_padded_qk_stride(name, w, stride):
    """q/k rows padded to `stride` (the 96 -> 128 case an attention kernel with
    equal head widths needs; 64 and 128 wide heads through the fused forward
    too; 48 -> 64 goes through the other norm/RoPE kernels): the first d_qk
    columns and every backward output are bit-equal to the unpadded run's,
    the padding is written as zeros, and the NaN bits in the padding of
    dq/dk are never read."""
    d = w["d_qk"]
    a = run(w, seed=13)
    b = run(w, seed=13, dy=a["dy"], qk_stride=stride)
    for key in ("q", "k"):
        assert b[key].shape[-1] == stride
        assert np.array_equal(b[key][..., :d], a[key]), key
        assert not b[key][..., d:].any(), key  # +0.0 bits, not NaN
    for key in ("v", "rho", "dqkv", "g_scales", "g8", "dx", "dw"):
        assert np.array_equal(a[key], b[key]), key
    if a["qk_pre"] is not None:
        assert np.array_equal(a["qk_pre"], b["qk_pre"])
    assert b["status"] == 0


@pytest.mark.parametrize("name,w", [("tiny", inputs.WORKLOADS["tiny"]), ("tails", TAILS)])
def test_e5m2_gradients_stagewise(name, w):
    """The backward with the packed gradient in e5m2: its codes and scale
    bit-exact, dX and dW (e5m2 x e4m3 on the matrix cores) to the GEMM bars;
    the forward is unchanged."""
    r = run(w, seed=21, grad_format=1)
    _check_forward(w, r)
    _check_backward(w, r, fmt="e5m2")
    assert r["status"] == 0
    # the e5m2 scale is amax / 57344
    g = bf16_to_f64(r["dqkv"])
    assert r["g_scales"][0] == np.float32(np.float32(np.abs(g).max()) / np.float32(57344.0))


def test_e5m2_gradients_end_to_end():
    """From the inputs alone: dX and dW with e5m2 gradients no further from
    the unquantised float64 gradients than 1.1x the oracle's own e5m2 chain
    + 1e-3, and e5m2 (2 fraction bits) measurably coarser than e4m3."""
    w = inputs.WORKLOADS["tiny"]
    r5 = run(w, seed=8, grad_format=1)
    r4 = run(w, seed=8)
    dims = _dims(w)
    ref_dx, ref_dw = _unquantised(w, r5["x_bits"], r5["W"], r5["dy"])
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, r5["W"])
    of = oracle.qkv_forward(dims, w["n_seq"], w["seq_len"], r5["x_bits"], wp, s_w)
    nqk2 = 2 * w["n_heads"] * w["d_qk"]
    dq, dk, dv = r5["dy"]
    ob = oracle.qkv_backward(dims, w["n_seq"], w["seq_len"], dq, dk, dv, of["x8"], of["s_x"],
                             of["y_bits"][:, :nqk2], wp, s_w, grad_fmt="e5m2")

    def err(a, b):
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    e_dx, e_dw = err(bf16_to_f64(r5["dx"]), ref_dx), err(r5["dw"], ref_dw)
    o_dx, o_dw = err(bf16_to_f64(ob["dx_bits"]), ref_dx), err(ob["dw64"], ref_dw)
    e4_dw = err(r4["dw"], ref_dw)
    say(f"[gpu] e5m2 e2e: dx gpu {e_dx:.3e} oracle {o_dx:.3e}; dw gpu {e_dw:.3e} oracle "
        f"{o_dw:.3e}; e4m3 dw {e4_dw:.3e}")
    assert e_dx <= 1.1 * o_dx + 1e-3 and e_dw <= 1.1 * o_dw + 1e-3
    assert e_dw > e4_dw


def test_zero_inputs_give_zero_outputs():
    w = RAGGED
    T = w["n_seq"] * w["seq_len"]
    x_bits = np.zeros((T, w["d_model"]), dtype=np.uint16)
    dq, dk, dv = inputs.make_dy(w, 1)
    dy = (np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv))
    r = run(w, seed=1, x_bits=x_bits, dy=dy)
    assert r["x_scales"][0] == 1.0 and r["g_scales"][0] == 1.0
    for key in ("q", "k", "v", "dx"):
        assert not (bf16_to_f64(r[key]) != 0).any(), key
    assert not (r["dw"] != 0).any()
    assert r["status"] == 0


def test_nonfinite_activation_sets_status():
    w = RAGGED
    x_bits = inputs.make_x(w, 2)
    x_bits[17, 3] = 0x7FC0  # NaN
    r = run(w, seed=2, x_bits=x_bits, backward=False)
    assert r["status"] & 2


# ------------------------------------------- the 64k-token step, sampled

def _direct_rel(gpu_bits, exact):
    """Worst row of ||gpu - round_bf16(exact)|| / ||round_bf16(exact)||: the
    GEMM bar read literally, against the bf16-rounded oracle."""
    return row_rel_err(bf16_to_f64(gpu_bits), bf16_to_f64(oracle.round_bf16(exact)))


@pytest.mark.parametrize("name,wl,fmt,qs", [
    ("tiny", inputs.WORKLOADS["tiny"], 0, 0), ("ragged", RAGGED, 0, 0),
    ("d64", dict(RAGGED, d_qk=64), 0, 0), ("d128", dict(RAGGED, d_qk=128), 0, 0),
    ("e5m2", RAGGED, 1, 0), ("padded", RAGGED, 0, 136),
    ("step_64k", inputs.WORKLOADS["step_64k"], 0, 0)])
def test_two_pass_backward_matches_one_pass(name, wl, fmt, qs):
    """The backward with the norm/RoPE backward fused into the gradient
    quantiser (two passes, no dQK in memory) writes the codes the one-pass
    form quantises from dQK, bit for bit, including the zero rows of the dW
    K tail, and so the same scale, dX and dW (also with padded q/k rows,
    whose NaN padding neither form may read)."""
    one = run(wl, seed=17, grad_format=fmt, qk_stride=qs)
    two = run(wl, seed=17, grad_format=fmt, qk_stride=qs, bwd_passes=2)
    assert two["dqkv"] is None
    for key in ("g8", "g8_kpad", "g8_tail", "g_scales", "dx", "q", "k", "v"):
        assert np.array_equal(one[key], two[key]), key
    assert np.array_equal(one["dw"].view(np.uint32), two["dw"].view(np.uint32))
    assert one["status"] == two["status"] == 0


@pytest.mark.parametrize("name,wl,qs,fmt,passes", [
    ("tiny", inputs.WORKLOADS["tiny"], 0, 0, 0), ("ragged", RAGGED, 0, 0, 0),
    ("d48", dict(RAGGED, d_qk=48), 0, 0, 0), ("d128", dict(RAGGED, d_qk=128), 0, 0, 0),
    ("padded", RAGGED, 136, 0, 0), ("e5m2", RAGGED, 0, 1, 0), ("two_pass", RAGGED, 0, 0, 2),
    ("step_64k", inputs.WORKLOADS["step_64k"], 0, 0, 0)])
def test_pack_forward_matches_separate_calls(name, wl, qs, fmt, passes):
    """qkv_pack_forward (the weight pack and the forward with their
    quantiser launches shared) writes what pack_quantize_weights followed by
    qkv_forward writes, bit for bit: both weight views and their scales, x8
    with its zero K and token tails and its scales, 1/rms, q, k, v; the
    backward from its cache and saved buffer then matches too; and it
    clears the status word it was handed with every bit set (also with e5m2
    gradients and the two-pass backward after it)."""
    sep = run(wl, seed=23, qk_stride=qs, grad_format=fmt, bwd_passes=passes)
    one = run(wl, seed=23, qk_stride=qs, grad_format=fmt, bwd_passes=passes, pack_forward=True)
    for key in ("w_packed", "w_packed_t", "w_scales", "x8", "x8_kpad", "x8_tail", "x_scales",
                "rho", "q", "k", "v", "g8", "g_scales", "dx"):
        assert np.array_equal(sep[key], one[key]), key
    assert np.array_equal(sep["dw"].view(np.uint32), one["dw"].view(np.uint32))
    assert sep["status"] == one["status"] == 0


def test_pack_forward_status_bits():
    """A NaN in W and one in x set the weight and the activation bits in
    the combined call as they do in the separate calls."""
    w = RAGGED
    x_bits = inputs.make_x(w, 4)
    x_bits[5, 7] = 0x7FC0
    W = inputs.make_w(w, 5)
    W[3, 11] = np.nan
    sep = run(w, seed=4, x_bits=x_bits, W=W, backward=False)
    one = run(w, seed=4, x_bits=x_bits, W=W, backward=False, pack_forward=True)
    assert sep["status"] == one["status"] == 3


@pytest.mark.parametrize("wl,fmt", [("step_64k", "e4m3"), ("sweep_64", "e4m3"),
                                    ("sweep_128", "e4m3"), ("step_64k", "e5m2")])
def test_step_64k_sampled_rows(wl, fmt):
    """Full-size forward + backward in the benchmark's launch configuration
    (the 96-wide heads, both other widths of the sweep, and the e5m2
    gradients): every FP8 code checked in full, the float outputs on
    sampled token rows (both ends included) and sampled dW rows.  At these
    K (768 for the projection, N for dX) the GEMM rows must also meet the
    1e-3 bar directly against the bf16-rounded oracle."""
    w = inputs.WORKLOADS[wl]
    dims = _dims(w)
    r = run(w, seed=42, grad_format=1 if fmt == "e5m2" else 0)
    T, H, dqk, dv, S = r["T"], w["n_heads"], w["d_qk"], w["d_v"], w["seq_len"]
    nq = H * dqk
    assert r["status"] == 0
    wp, wpt, s_w, inv_w, _ = oracle.pack_quantize_weights(dims, r["W"])
    assert np.array_equal(r["w_packed"], wp) and np.array_equal(r["w_packed_t"], wpt)
    x8, s_x, inv_x, _ = oracle.quantize_bf16(r["x_bits"])
    assert np.array_equal(r["x8"], x8) and r["x_scales"][0] == s_x
    assert not r["x8_tail"].any()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, 253, replace=False)]))
    pos = rows % S
    # GEMM rows: the V columns (and the stored pre-norm rows, if any)
    y64 = oracle.gemm_e4m3(x8[rows], wp, s_x, s_w)
    gpu_v = r["v"][0][:, rows, :].transpose(1, 0, 2).reshape(len(rows), -1)
    _, over_gemm = bf16_gemm_excess(gpu_v, y64[:, 2 * nq:], oracle.round_bf16)
    d_gemm = _direct_rel(gpu_v, y64[:, 2 * nq:])
    if r["qk_pre"] is not None:
        _, over_qk = bf16_gemm_excess(r["qk_pre"][rows], y64[:, :2 * nq], oracle.round_bf16)
        over_gemm = max(over_gemm, over_qk)
        d_gemm = max(d_gemm, _direct_rel(r["qk_pre"][rows], y64[:, :2 * nq]))
    # norm/RoPE rows, fed the pre-norm values
    a_bits = _prenorm_bits(w, r, rows)
    a = bf16_to_f64(a_bits)
    qo = oracle.qk_norm_rope_fwd(a[:, :nq].reshape(-1, H, dqk), pos, EPS, BASE)
    ko = oracle.qk_norm_rope_fwd(a[:, nq:].reshape(-1, H, dqk), pos, EPS, BASE)
    e_q = row_rel_err(bf16_to_f64(r["q"][0][:, rows, :].transpose(1, 0, 2)), qo)
    e_k = row_rel_err(bf16_to_f64(r["k"][0][:, rows, :].transpose(1, 0, 2)), ko)
    over_rho, e_rho = _rho_excess(rho_rows(r["rho"])[rows], y64[:, :2 * nq], H, dqk)
    # backward norm/RoPE rows (the oracle from the pre-norm rows)
    dq, dk, dvg = r["dy"]
    dqo = oracle.qk_norm_rope_bwd(a[:, :nq].reshape(-1, H, dqk),
                                  bf16_to_f64(dq[0][:, rows, :].transpose(1, 0, 2)), pos, EPS, BASE)
    dko = oracle.qk_norm_rope_bwd(a[:, nq:].reshape(-1, H, dqk),
                                  bf16_to_f64(dk[0][:, rows, :].transpose(1, 0, 2)), pos, EPS, BASE)
    gq = bf16_to_f64(r["dqkv"][rows, :nq]).reshape(-1, H, dqk)
    gk = bf16_to_f64(r["dqkv"][rows, nq:2 * nq]).reshape(-1, H, dqk)
    e_dq = row_rel_err(gq, dqo)
    e_dk = row_rel_err(gk, dko)
    assert np.array_equal(r["dqkv"][rows, 2 * nq:],
                          dvg[0][:, rows, :].transpose(1, 0, 2).reshape(len(rows), -1))
    # gradient codes in full
    g8, s_g, inv_g, _ = oracle.quantize_bf16(r["dqkv"], fmt)
    assert np.array_equal(r["g8"], g8) and r["g_scales"][0] == s_g
    assert not r["g8_tail"].any()
    # dX rows and dW rows
    dx64 = oracle.gemm_e4m3(g8[rows], np.ascontiguousarray(wp.T), s_g, s_w, a_fmt=fmt)
    d_dx = _direct_rel(r["dx"][rows], dx64)
    _, over_dx = bf16_gemm_excess(r["dx"][rows], dx64, oracle.round_bf16)
    jrows = np.unique(np.concatenate([[0, w["d_model"] - 1], rng.choice(w["d_model"], 30)]))
    dw = oracle.round_f32(oracle.gemm_e4m3(np.ascontiguousarray(x8[:, jrows].T), g8, s_x, s_g,
                                           b_fmt=fmt))
    e_dw = row_rel_err(r["dw"][jrows], dw)
    say(f"[gpu] {wl} {fmt}: gemm direct {d_gemm:.2e} (excess {over_gemm:.2e}) q {e_q:.2e} "
        f"k {e_k:.2e} rho {e_rho:.2e} dq {e_dq:.2e} dk {e_dk:.2e} dx direct {d_dx:.2e} "
        f"(excess {over_dx:.2e}) dw {e_dw:.2e}")
    assert over_gemm <= GEMM_TOL and over_dx <= GEMM_TOL and e_dw <= GEMM_TOL
    assert d_gemm <= GEMM_TOL and d_dx <= GEMM_TOL  # the literal bar
    assert over_rho <= GEMM_TOL
    assert max(e_q, e_k, e_dq, e_dk) <= NORM_TOL


# ------------------------------------------- exact GEMMs (integer inputs)

def _int_values(rng, shape):
    return rng.integers(-2, 3, size=shape).astype(np.float32)


def test_gemms_bit_exact_on_integer_inputs():
    """Small integers plus one 448 in each tensor make every scale exactly 1,
    every code exact and every product sum an integer far below 2^14, so the
    forward projection, dX and dW must equal the oracle's bit for bit
    (integer brute force through the whole C interface)."""
    w = dict(n_seq=2, seq_len=192, d_model=256, n_heads=2, d_qk=96, d_v=128)
    dims = _dims(w)
    n_seq, S, D, H = w["n_seq"], w["seq_len"], w["d_model"], w["n_heads"]
    T, N, nq = n_seq * S, inputs.packed_width(w), H * w["d_qk"]
    rng = np.random.default_rng(7)
    x = _int_values(rng, (T, D))
    x[0, 0] = 448.0
    W = _int_values(rng, (D, N))
    W[1, 0] = 448.0
    dv = _int_values(rng, (n_seq, H, S, w["d_v"]))
    dv[0, 0, 1, 0] = 448.0  # token 1: its x row holds no 448
    zero = np.zeros((n_seq, H, S, w["d_qk"]), dtype=np.float32)
    dy = tuple(inputs.f32_to_bf16_bits(a) for a in (zero, zero, dv))
    r = run(w, seed=7, x_bits=inputs.f32_to_bf16_bits(x), W=W, dy=dy)
    assert r["status"] == 0
    assert r["x_scales"][0] == 1.0 and r["w_scales"][0] == 1.0 and r["g_scales"][0] == 1.0
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, W)
    x8, s_x, _, _ = oracle.quantize_bf16(r["x_bits"])
    y = oracle.round_bf16(oracle.gemm_e4m3(x8, wp, s_x, s_w))
    assert r["fused"]  # d_qk = 96: the norm/RoPE epilogue of the GEMM
    assert np.array_equal(r["v"], oracle.to_head_major(y[:, 2 * nq:].reshape(T, H, -1), n_seq, S))
    # the exact Q|K products through the fused norm/RoPE: each element within
    # the bf16 rounding of the output (2^-8 relative of the row's largest)
    o = oracle.qkv_forward(dims, n_seq, S, r["x_bits"], wp, s_w, y_bits=y)
    for key in ("q", "k"):
        got, want = bf16_to_f64(r[key]), o[key + "64"]
        bound = 2.0 ** -8 * np.abs(want).max(axis=-1, keepdims=True)
        assert np.all(np.abs(got - want) <= bound), key
    # zero upstream q, k gradients: dQKV = [0 | dv]
    assert not bf16_to_f64(r["dqkv"][:, :2 * nq]).any()  # zeros of either sign
    g8, s_g, _, _ = oracle.quantize_bf16(r["dqkv"])
    dx = oracle.round_bf16(oracle.gemm_e4m3(g8, np.ascontiguousarray(wp.T), s_g, s_w))
    assert np.array_equal(r["dx"], dx)
    dw = oracle.round_f32(oracle.gemm_e4m3(np.ascontiguousarray(x8.T), g8, s_x, s_g))
    assert np.array_equal(r["dw"], dw)


def test_all_codes_through_the_forward_gemm():
    """x holds every finite e4m3 value (scale 1: 448 is among them) and W is
    the identity in the V columns plus one 448 that fixes its scale at 1: v
    is the decoded codes themselves, so the matrix cores' reading of every
    code, subnormals included, is checked bit for bit."""
    w = inputs.WORKLOADS["tiny"]
    dims = _dims(w)
    T, D, N = w["n_seq"] * w["seq_len"], w["d_model"], inputs.packed_width(w)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(np.resize(codes, T * D)).reshape(T, D).astype(np.float32)
    x_bits = inputs.f32_to_bf16_bits(vals)
    assert np.array_equal(oracle.bf16_to_f64(x_bits), vals)  # every e4m3 value is a bf16 value
    nqk2 = 2 * w["n_heads"] * w["d_qk"]
    assert N - nqk2 == D  # the V columns hold the identity
    W = np.zeros((D, N), dtype=np.float32)
    W[np.arange(D), nqk2 + np.arange(D)] = 1.0
    W[0, 0] = 448.0
    r = run(w, seed=7, x_bits=x_bits, W=W, backward=False)
    assert r["x_scales"][0] == 1.0 and r["w_scales"][0] == 1.0
    assert np.array_equal(r["x8"], np.resize(codes, T * D).reshape(T, D))
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, W)
    y = oracle.round_bf16(oracle.gemm_e4m3(r["x8"], wp, 1.0, s_w))
    gpu_v = oracle.from_head_major(r["v"]).reshape(T, -1)
    assert np.array_equal(gpu_v, y[:, nqk2:])
    # the identity columns reproduce the decode table (signed zeros add to +0)
    assert np.array_equal(oracle.bf16_to_f64(gpu_v), vals + 0.0)


# ------------------------------------------------ the largest token count

def _gather_blocked_rows(buf, off, rows, cols, lay):
    """Rows of a blocked FP8 copy inside a device byte buffer, gathered on the
    device: [len(rows)][ceil(cols / k_block) * k_block] uint8 on the host."""
    R, KB = lay.act_block_rows, lay.k_block
    kc = -(-cols // KB)
    t = torch.as_tensor(rows, dtype=torch.int64, device=buf.device)
    kb = torch.arange(kc, device=buf.device)
    c = torch.arange(KB, device=buf.device)
    idx = (off + (((t // R)[:, None] * kc + kb[None, :]) * R + (t % R)[:, None])[:, :, None] * KB
           + c[None, None, :])
    return buf[idx.reshape(-1)].reshape(len(rows), kc * KB).cpu().numpy()


def _gather_blocked_column(buf, off, col, T, cols, lay):
    """One column (all T rows) of a blocked FP8 copy, gathered on the device."""
    R, KB = lay.act_block_rows, lay.k_block
    kc = -(-cols // KB)
    t = torch.arange(T, dtype=torch.int64, device=buf.device)
    idx = off + (((t // R) * kc + col // KB) * R + t % R) * KB + col % KB
    return buf[idx].cpu().numpy()


def test_max_tokens_sampled():
    """The largest supported token count, T = 2^24 (256 sequences of 65536
    positions), at the tiny workload's widths (D = 128, one head), so that
    every tensor fits: the offsets that this token cap is there to keep in
    range are exercised at their limit.  Inputs come from torch's seeded
    generator on the device (x ~ N(0,1), dq/dk/dv ~ N(0, 1e-2)); the oracle
    gets the same values copied to the host.  Checked: both scales against
    the oracle's quantiser of the whole tensor's amax; sampled token rows of
    x8, q, k, v, the gradient codes and dX against the oracle; dW entries
    (sums over all 2^24 tokens) to 1e-3 of their natural scale sqrt(sum of
    squared terms); and qkv_pack_forward's outputs equal to those of the two
    separate calls, byte for byte."""
    from fp8_packed_reduced_amd import binding as B
    w = dict(inputs.WORKLOADS["tiny"], n_seq=256, seq_len=65536)
    n_seq, S, D, H, dqk, dvw = (w[k] for k in ("n_seq", "seq_len", "d_model", "n_heads",
                                                "d_qk", "d_v"))
    T, nq = n_seq * S, H * dqk
    assert T == 1 << 24
    dims_o = _dims(w)
    dims = B.make_dims(D, H, dqk, dvw, EPS, BASE)
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    say(f"[gpu] max tokens: T={T} D={D} H={H}")
    x = torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16)
    dq = (torch.randn((n_seq, H, S, dqk), generator=g, device=dev) * 0.1).to(torch.bfloat16)
    dk = (torch.randn((n_seq, H, S, dqk), generator=g, device=dev) * 0.1).to(torch.bfloat16)
    dv = (torch.randn((n_seq, H, S, dvw), generator=g, device=dev) * 0.1).to(torch.bfloat16)
    W = inputs.make_w(w, 43)
    Wd = torch.from_numpy(W).to(dev)
    cache = B.WeightCache(dims)
    B.pack_quantize_weights(dims, Wd[:, :nq], Wd[:, nq:2 * nq], Wd[:, 2 * nq:], cache)
    saved = torch.zeros(B.saved_bytes(dims, T), dtype=torch.uint8, device=dev)
    q, k, v, saved = B.qkv_forward(dims, n_seq, S, x, cache, saved=saved)
    # the weight pack and the forward in one call, into fresh buffers: the
    # same bytes (its launches' grids are largest at this token count)
    cache2 = B.WeightCache(dims)
    saved2 = torch.zeros_like(saved)
    q2, k2, v2, _ = B.qkv_pack_forward(dims, Wd[:, :nq], Wd[:, nq:2 * nq], Wd[:, 2 * nq:], cache2,
                                       n_seq, S, x, saved=saved2)
    torch.cuda.synchronize()
    for a, b_, name in ((q, q2, "q"), (k, k2, "k"), (v, v2, "v"), (saved, saved2, "saved"),
                        (cache.w_packed, cache2.w_packed, "w_packed"),
                        (cache.w_packed_t, cache2.w_packed_t, "w_packed_t"),
                        (cache.scales, cache2.scales, "w_scales"),
                        (cache.status, cache2.status, "status")):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b_.view(torch.uint8) if b_.dtype == torch.bfloat16 else b_), name
    del q2, k2, v2, saved2, cache2
    ws_b = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_BACKWARD), dtype=torch.uint8,
                       device=dev)
    dx, dw = B.qkv_backward(dims, n_seq, S, q, k, dq, dk, dv, saved, cache, workspace=ws_b)
    torch.cuda.synchronize()
    say("[gpu] max tokens: run done")
    lay = B.layout(dims, T)
    assert int(cache.status.item()) == 0
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims_o, W)
    assert np.array_equal(cache.w_packed.cpu().numpy(), wp)

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def amax_scales(*arrays):
        m = max(int((a & 0x7FFF).max()) for a in arrays)  # |bf16| bit patterns are ordered
        _, s, inv, _ = oracle.quantize_bf16(np.array([m], np.uint16))
        return s, inv

    x_h = bits(x)
    s_x, inv_x = amax_scales(x_h)
    xsc = B.view_bytes(saved, lay.saved_x_scales, (2,), torch.float32).cpu().numpy()
    assert xsc[0] == s_x and xsc[1] == inv_x
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, S - 1, S, T - S, T - 2, T - 1],
                                     rng.choice(T, 57, replace=False)]))
    pos = rows % S
    x8r = _gather_blocked_rows(saved, lay.saved_x8, rows, D, lay)[:, :D]
    assert np.array_equal(x8r, oracle.e4m3_encode(oracle.bf16_to_f64(x_h[rows]) * inv_x))
    # forward rows: the oracle's GEMM and norm/RoPE of these tokens
    y64 = oracle.gemm_e4m3(x8r, wp, s_x, s_w)
    assert lay.fused_forward  # the pre-norm rows are the oracle's product of the codes
    qkr = oracle.round_bf16(y64[:, :2 * nq])
    rho_g = B.view_bytes(saved, lay.saved_rho, (2, n_seq, H, S), torch.float32)
    rho_r = rho_g[:, torch.as_tensor(rows // S, device=dev), :, torch.as_tensor(rows % S, device=dev)]
    rho_r = rho_r.cpu().numpy()  # [rows][2][H]
    over_rho, e_rho = _rho_excess(rho_r.reshape(len(rows), 2 * H), y64[:, :2 * nq], H, dqk)
    a = bf16_to_f64(qkr)
    qo = oracle.qk_norm_rope_fwd(a[:, :nq].reshape(-1, H, dqk), pos, EPS, BASE)
    ko = oracle.qk_norm_rope_fwd(a[:, nq:].reshape(-1, H, dqk), pos, EPS, BASE)
    b_idx, s_idx = torch.as_tensor(rows // S, device=dev), torch.as_tensor(pos, device=dev)
    e_q = row_rel_err(bf16_to_f64(bits(q[b_idx, :, s_idx])), qo)
    e_k = row_rel_err(bf16_to_f64(bits(k[b_idx, :, s_idx])), ko)
    vr = bits(v[b_idx, :, s_idx]).reshape(len(rows), -1)
    _, over_v = bf16_gemm_excess(vr, y64[:, 2 * nq:], oracle.round_bf16)
    # gradient scale from the whole dQKV; gradient codes and dX on the rows
    dqkv = B.view_bytes(ws_b, lay.bwd_dqkv, (T, 2 * nq), torch.bfloat16)
    s_g, inv_g = amax_scales(bits(dqkv), bits(dv))
    gsc = B.view_bytes(ws_b, lay.bwd_g_scales, (2,), torch.float32).cpu().numpy()
    assert gsc[0] == s_g and gsc[1] == inv_g
    N = 2 * nq + H * dvw
    g8r = _gather_blocked_rows(ws_b, lay.bwd_g8, rows, N, lay)[:, :N]
    gr = np.concatenate([bits(dqkv[torch.as_tensor(rows, device=dev)]),
                         bits(dv[b_idx, :, s_idx]).reshape(len(rows), -1)], axis=1)
    assert np.array_equal(g8r, oracle.e4m3_encode(oracle.bf16_to_f64(gr) * inv_g))
    dx64 = oracle.gemm_e4m3(g8r, np.ascontiguousarray(wp.T), s_g, s_w)
    _, over_dx = bf16_gemm_excess(bits(dx[torch.as_tensor(rows, device=dev)]), dx64,
                                  oracle.round_bf16)
    # dW entries over all tokens
    tab = oracle.e4m3_decode_table()
    dw_h = dw.cpu().numpy()
    worst = 0.0
    for j in (0, D - 1):
        xc = tab[_gather_blocked_column(saved, lay.saved_x8, j, T, D, lay)]
        for n in (0, nq, 2 * nq, N - 1):
            terms = xc * tab[_gather_blocked_column(ws_b, lay.bwd_g8, n, T, N, lay)]
            exact = float(s_x) * float(s_g) * terms.sum()
            scale = float(s_x) * float(s_g) * np.sqrt(np.sum(terms * terms))
            worst = max(worst, abs(float(dw_h[j, n]) - exact) / scale)
    say(f"[gpu] max tokens: rho {e_rho:.2e} v {over_v:.2e} q {e_q:.2e} k {e_k:.2e} "
        f"dx excess {over_dx:.2e} dw {worst:.2e}")
    assert over_v <= GEMM_TOL and over_dx <= GEMM_TOL and over_rho <= GEMM_TOL
    assert max(e_q, e_k) <= NORM_TOL and worst <= GEMM_TOL
