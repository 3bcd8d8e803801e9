"""qkv_forward_noalloc, the forward for callers that cannot allocate (its
workspace is the library's fixed per-device scratch), against qkv_forward
with a caller-allocated workspace: bit-identical q, k, v and saved state on
two calls in a row, the second with fewer tokens (the scratch keeps the
first call's contents).  Through the C interface."""
import numpy as np
import pytest
import torch

from fp8_packed_reduced_amd import binding as B
from fp8_packed_reduced_amd import inputs

from gpu_run import EPS, BASE, bits_to_dev, dev_to_bits, say, unblock_rows

pytestmark = pytest.mark.gpu


def _forward_both(w, seed):
    n_seq, S = w["n_seq"], w["seq_len"]
    T, D, H, dqk, dv = n_seq * S, w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
    nq = H * dqk
    say(f"[gpu] noalloc n_seq={n_seq} S={S} D={D} H={H} d_qk={dqk} seed={seed}")
    dims = B.make_dims(D, H, dqk, dv, EPS, BASE)
    W = torch.from_numpy(inputs.make_w(w, seed + 1)).cuda()
    cache = B.WeightCache(dims)
    B.pack_quantize_weights(dims, W[:, :nq], W[:, nq:2 * nq], W[:, 2 * nq:], cache)
    x = bits_to_dev(inputs.make_x(w, seed))
    ref = B.qkv_forward(dims, n_seq, S, x, cache)
    nan = lambda t: torch.full_like(t.view(torch.int16), -1).view(torch.bfloat16)
    q, k, v = nan(ref[0]), nan(ref[1]), nan(ref[2])
    saved = torch.full_like(ref[3], 0xAB)
    B.qkv_forward_noalloc(dims, n_seq, S, x, cache, q, k, v, saved)
    torch.cuda.synchronize()
    lay = B.layout(dims, T)
    for name, a, b in (("q", ref[0], q), ("k", ref[1], k), ("v", ref[2], v)):
        assert np.array_equal(dev_to_bits(a), dev_to_bits(b)), name
    # saved state: x8 (with its zero K tail rows), 1/rms per Q/K row, scales
    xa = unblock_rows(ref[3], lay.saved_x8, T, D, lay)[:lay.tokens_padded]
    xb = unblock_rows(saved, lay.saved_x8, T, D, lay)[:lay.tokens_padded]
    assert np.array_equal(xa, xb)
    for off, shape, dt in ((lay.saved_rho, (2 * T * H,), torch.float32),
                           (lay.saved_x_scales, (2,), torch.float32)):
        assert torch.equal(B.view_bytes(ref[3], off, shape, dt), B.view_bytes(saved, off, shape, dt))
    assert int(cache.status.item()) == 0
    return dims, cache, q, k, saved


def test_noalloc_forward_matches_two_calls_in_a_row():
    assert B.noalloc_scratch_bytes() == 64 * 1024
    big = dict(n_seq=3, seq_len=1000, d_model=768, n_heads=6, d_qk=96, d_v=128)
    small = dict(n_seq=1, seq_len=77, d_model=768, n_heads=6, d_qk=96, d_v=128)
    _forward_both(big, 31)
    _forward_both(small, 32)


def test_noalloc_forward_feeds_the_backward():
    w = dict(n_seq=2, seq_len=300, d_model=256, n_heads=2, d_qk=64, d_v=128)
    dims, cache, q, k, saved = _forward_both(w, 33)
    n_seq, S = w["n_seq"], w["seq_len"]
    dq, dk, dvg = (bits_to_dev(a) for a in inputs.make_dy(w, 35))
    dx, dw = B.qkv_backward(dims, n_seq, S, q, k, dq, dk, dvg, saved, cache)
    torch.cuda.synchronize()
    assert torch.isfinite(dx.float()).all() and torch.isfinite(dw).all()


def test_noalloc_forward_refuses_what_the_scratch_cannot_hold():
    # d_qk = 48 has no fused forward: its pre-norm rows would need the
    # workspace, far beyond the fixed scratch; refused before any launch
    dims = B.make_dims(192, 2, 48, 64, EPS, BASE)
    assert B.workspace_bytes(dims, 4096, B.FPR_CALL_FORWARD) > B.noalloc_scratch_bytes()
    cache = B.WeightCache(dims)
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    x, q, k, v = z(4096, 192), z(1, 2, 4096, 48), z(1, 2, 4096, 48), z(1, 2, 4096, 64)
    saved = torch.zeros(B.saved_bytes(dims, 4096), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.FprError) as err:
        B.qkv_forward_noalloc(dims, 1, 4096, x, cache, q, k, v, saved)
    assert err.value.code == 6
