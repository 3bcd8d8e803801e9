"""The library's calls only enqueue kernels on the caller's stream (no
allocation, memset or synchronisation), so a whole step can be captured in a
HIP graph and replayed.  Each replay must reproduce the eager outputs bit for
bit; before every replay the outputs are overwritten with NaN and unrelated
eager work runs, with synchronisations in between."""
import numpy as np
import pytest
import torch

from fp8_packed_reduced_amd import binding as B
from fp8_packed_reduced_amd import inputs

from gpu_run import bits_to_dev, dims_for, say

pytestmark = pytest.mark.gpu

QKV = dict(n_seq=3, seq_len=100, d_model=128, n_heads=2, d_qk=96, d_v=128)
MLP = dict(n_seq=1, seq_len=333, d_model=192, d_ff=320)
REPLAYS = 3


def _snapshot(ts):
    return [t.detach().clone().view(torch.uint8).cpu().numpy() for t in ts]


def _scribble(ts):
    for t in ts:
        if t.dtype in (torch.bfloat16, torch.float32):
            t.fill_(float("nan"))
        else:
            t.fill_(0x7F)


def _replay_and_check(graph, outs, want, name):
    for r in range(REPLAYS):
        _scribble(outs)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(outs)
        for i, (g, w) in enumerate(zip(got, want)):
            assert np.array_equal(g, w), (name, r, i)
        say(f"[gpu] graph {name}: replay {r} matches ({float(junk):.1f})")


def test_qkv_step_replays_from_a_graph():
    w = QKV
    n_seq, S = w["n_seq"], w["seq_len"]
    T, D, H, dqk, dv = n_seq * S, w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
    nq, N = H * dqk, inputs.packed_width(w)
    dims = dims_for(w)
    x = bits_to_dev(inputs.make_x(w, 5))
    W = torch.from_numpy(inputs.make_w(w, 6)).cuda()
    dq, dk, dvg = (bits_to_dev(a) for a in inputs.make_dy(w, 7))
    cache = B.WeightCache(dims)
    ws_p = torch.empty(B.workspace_bytes(dims, 0, B.FPR_CALL_PACK), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_FORWARD), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_BACKWARD), dtype=torch.uint8,
                       device="cuda")
    saved = torch.empty(B.saved_bytes(dims, T), dtype=torch.uint8, device="cuda")
    q = torch.empty((n_seq, H, S, dqk), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((n_seq, H, S, dv), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((D, N), dtype=torch.float32, device="cuda")

    def step():
        B.pack_quantize_weights(dims, W[:, :nq], W[:, nq:2 * nq], W[:, 2 * nq:], cache,
                                workspace=ws_p)
        B.qkv_forward(dims, n_seq, S, x, cache, q, k, v, saved, ws_f)
        B.qkv_backward(dims, n_seq, S, q, k, dq, dk, dvg, saved, cache, dx, dw, ws_b)

    outs = [cache.w_packed, cache.w_packed_t, cache.scales, q, k, v, dx, dw]
    step()
    torch.cuda.synchronize()
    want = _snapshot(outs)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    _replay_and_check(graph, outs, want, "qkv")
    assert int(cache.status.item()) == 0


def test_mlp_step_replays_from_a_graph():
    w = MLP
    T, D, F = w["n_seq"] * w["seq_len"], w["d_model"], w["d_ff"]
    dims = B.MlpDims(D, F)
    x = bits_to_dev(inputs.make_x(w, 8))
    w1, w2 = (torch.from_numpy(a).cuda() for a in inputs.make_mlp_w(w, 9))
    dy = bits_to_dev(inputs.make_mlp_dy(w, 10))
    cache = B.MlpCache(dims)
    ws_p = torch.empty(B.mlp_workspace_bytes(dims, 0, B.FPR_CALL_PACK), dtype=torch.uint8,
                       device="cuda")
    ws_f = torch.empty(B.mlp_workspace_bytes(dims, T, B.FPR_CALL_FORWARD), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(B.mlp_workspace_bytes(dims, T, B.FPR_CALL_BACKWARD), dtype=torch.uint8,
                       device="cuda")
    saved = torch.empty(B.mlp_saved_bytes(dims, T), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    dw1 = torch.empty((D, F), dtype=torch.float32, device="cuda")
    dw2 = torch.empty((F, D), dtype=torch.float32, device="cuda")

    def step():
        B.mlp_pack_quantize_weights(dims, w1, w2, cache, workspace=ws_p)
        B.mlp_forward(dims, x, cache, y, saved, ws_f)
        B.mlp_backward(dims, dy, saved, cache, dx, dw1, dw2, ws_b)

    outs = [cache.w1, cache.w2_t, cache.scales, y, dx, dw1, dw2]
    step()
    torch.cuda.synchronize()
    want = _snapshot(outs)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    _replay_and_check(graph, outs, want, "mlp")
    assert int(cache.status.item()) == 0
