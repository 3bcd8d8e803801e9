"""Host-side checks of the C interface (no GPU needed, nothing is launched):
the library loads, exports every call the header declares, sizes and the
private layout are consistent, and every argument error is reported before
any kernel launch.  The argument-error tests pass made-up device addresses,
so they run only where no GPU is visible: there a check that regressed
could reach a launch on an unmapped address."""
import ctypes

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

from fp8_packed_reduced_amd import binding as B

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(B.LIB_PATH),
                                reason="libfpr.so not built")


def test_library_exports_every_declared_call():
    names = B.declared_functions()
    assert set(names) == {"fpr_workspace_bytes", "fpr_saved_bytes", "pack_quantize_weights",
                          "qkv_forward", "qkv_backward", "fpr_status_string", "fpr_get_layout",
                          "fpr_e4m3_encode", "fpr_trace_set", "fpr_mlp_workspace_bytes",
                          "fpr_mlp_saved_bytes", "fpr_mlp_get_layout",
                          "mlp_pack_quantize_weights", "mlp_forward", "mlp_backward",
                          "fpr_e5m2_encode", "qkv_forward_noalloc", "fpr_noalloc_scratch_bytes",
                          "fpr_probe_copy", "fpr_probe_read", "fpr_probe_mfma",
                          "qkv_pack_forward", "mlp_pack_forward"}
    lib = B.load()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(7):
        assert B.status_string(code)
    assert "unknown" in B.status_string(99)


def test_sizes_and_layout_at_the_64k_step_shape():
    d = B.make_dims(768, 6)
    T = 65536
    lay = B.layout(d, T)
    assert lay.tokens == T and lay.tokens_padded == T
    saved = B.saved_bytes(d, T)
    # x8 [T][768] blocked + 1/rms of 12 Q/K head rows per token + scales; no
    # pre-norm rows (the norm/RoPE runs in the GEMM's epilogue at d_qk = 96)
    assert lay.fused_forward
    assert 768 * T + T * 12 * 4 + 8 <= saved < 768 * T + T * 12 * 4 + 4096
    assert lay.saved_x8 + 768 * T <= lay.saved_rho
    assert lay.saved_rho + T * 12 * 4 <= lay.saved_x_scales < saved
    # the forward workspace holds only the x amax partials
    assert B.workspace_bytes(d, T, B.FPR_CALL_FORWARD) <= 4096
    bw = B.workspace_bytes(d, T, B.FPR_CALL_BACKWARD)
    assert bw >= lay.bwd_g8 + 1920 * T
    for off in (lay.saved_x8, lay.saved_rho, lay.saved_x_scales,
                lay.bwd_dqkv, lay.bwd_g8, lay.bwd_g_scales, lay.bwd_dw_part):
        assert off % 256 == 0
    # split-K partials of dW fit after the gradient codes
    assert 1 <= lay.dw_splits <= 8
    assert lay.bwd_dw_part >= lay.bwd_g8 + 1920 * T
    assert lay.bwd_dw_part + lay.dw_splits * 768 * 1920 * 4 <= bw
    # the pack + forward call's workspace: the pack's, aligned, then the forward's
    pk = B.workspace_bytes(d, 0, B.FPR_CALL_PACK)
    fw = B.workspace_bytes(d, T, B.FPR_CALL_FORWARD)
    assert pk + fw <= B.workspace_bytes(d, T, B.FPR_CALL_PACK_FORWARD) < pk + fw + 256


def test_blocked_fp8_layouts_cover_their_padding():
    # ragged everywhere: 154 tokens, D = 192, N = 2 * 2 * 48 + 2 * 64 = 320
    d = B.make_dims(192, 2, 48, 64)
    T = 154
    lay = B.layout(d, T)
    assert (lay.k_block, lay.act_block_rows) == (128, 256)
    assert lay.tokens_padded == 256
    # x8: one block row of 256 tokens x 2 K blocks of 128 bytes
    assert lay.saved_x8 + 256 * 256 <= lay.saved_rho
    # g8: 256 tokens x 3 K blocks
    assert lay.bwd_g8 + 256 * 384 <= lay.bwd_dw_part


def test_dw_split_count_depends_only_on_shapes():
    d = B.make_dims(768, 6)
    # 768 x 1920 in 256 x 128 tiles is 45 tiles; 5 splits make 225 blocks,
    # the fullest single round of 256 compute units with at most 8 splits
    assert B.layout(d, 65536).dw_splits == 5
    assert B.layout(d, 16384).dw_splits == 5
    # never more splits than 128-token K steps
    assert B.layout(B.make_dims(128, 1), 100).dw_splits == 1


def test_unfused_widths_keep_the_prenorm_rows_in_the_forward_workspace():
    # d_qk = 48: no fused forward; its pre-norm Q|K rows [T][2 * 2 * 48] bf16
    # pass through the forward workspace, never the saved buffer
    d = B.make_dims(192, 2, 48, 64)
    T = 1000
    lay = B.layout(d, T)
    assert not lay.fused_forward
    assert lay.fwd_qk_pre % 256 == 0
    assert lay.fwd_qk_pre + T * 192 * 2 <= B.workspace_bytes(d, T, B.FPR_CALL_FORWARD)
    for dqk in (64, 96, 128):
        assert B.layout(B.make_dims(768, 6, dqk, 128), T).fused_forward


@pytest.mark.parametrize("dims", [(768, 6, 96, 128), (192, 2, 48, 64), (128, 1, 96, 128)])
def test_amax_partials_stay_bounded(dims):
    # every quantiser block folds all partials of its tensor: their number
    # must not grow with the token count (at most 4096)
    d = B.make_dims(*dims)
    for T in (1, 1000, 65536, 1 << 24):
        lay = B.layout(d, T)
        assert 1 <= lay.bwd_amax_partials <= 1024 + 256


def test_token_limit():
    d = B.make_dims(768, 6)
    assert B.workspace_bytes(d, 1 << 24, B.FPR_CALL_BACKWARD) > 0
    assert B.workspace_bytes(d, (1 << 24) + 1, B.FPR_CALL_BACKWARD) == 0
    assert B.saved_bytes(d, (1 << 24) + 1) == 0


def test_ragged_tokens_pad_to_whole_k_steps():
    d = B.make_dims(128, 1)
    assert B.layout(d, 300).tokens_padded == 384
    assert B.layout(d, 1).tokens_padded == 128


@pytest.mark.parametrize("dims,ok", [
    ((768, 6, 96, 128), True), ((128, 1, 96, 128), True), ((768, 6, 64, 128), True),
    ((768, 6, 128, 128), True), ((100, 6, 96, 128), False), ((768, 6, 40, 128), False),
    ((768, 6, 96, 120), False), ((768, 1, 32, 32), False), ((768, 0, 96, 128), False),
    ((768, 16, 96, 128), True), ((4096, 32, 96, 128), True), ((768, 24, 48, 64), False),
    ((768, 65, 96, 128), False)])
def test_shape_support(dims, ok):
    d = B.make_dims(*dims)
    assert (B.saved_bytes(d, 256) > 0) == ok
    assert (B.workspace_bytes(d, 256, B.FPR_CALL_FORWARD) > 0) == ok


@pytest.mark.parametrize("stride,ok", [
    (0, True), (96, True), (128, True), (104, True), (1024, True), (88, False), (100, False),
    (1032, False), (-8, False)])
def test_qk_stride_support(stride, ok):
    d = B.make_dims(768, 6, 96, 128, qk_stride=stride)
    assert (B.saved_bytes(d, 256) > 0) == ok
    assert (B.workspace_bytes(d, 256, B.FPR_CALL_BACKWARD) > 0) == ok


def test_qk_stride_leaves_buffers_alone():
    """Padding only changes the caller's q/k/dq/dk rows, never the library's
    saved or workspace buffers."""
    a, b = B.make_dims(768, 6), B.make_dims(768, 6, qk_stride=128)
    assert B.saved_bytes(a, 4096) == B.saved_bytes(b, 4096)
    for which in (B.FPR_CALL_FORWARD, B.FPR_CALL_BACKWARD):
        assert B.workspace_bytes(a, 4096, which) == B.workspace_bytes(b, 4096, which)
    assert ctypes.sizeof(B.Dims) == 36 and B.Dims.qk_stride.offset == 24
    assert B.Dims.grad_format.offset == 28 and B.Dims.bwd_passes.offset == 32


@pytest.mark.parametrize("fmt,ok", [(0, True), (1, True), (2, False), (-1, False)])
def test_grad_format_support(fmt, ok):
    d = B.make_dims(768, 6, grad_format=fmt)
    assert (B.workspace_bytes(d, 256, B.FPR_CALL_BACKWARD) > 0) == ok
    if ok:  # the format changes no buffer size
        assert B.workspace_bytes(d, 4096, B.FPR_CALL_BACKWARD) == \
            B.workspace_bytes(B.make_dims(768, 6), 4096, B.FPR_CALL_BACKWARD)


def _cache_c(ptr=0x1000):
    return B._CacheC(ptr, ptr, ptr, ptr)


_NO_GPU = pytest.mark.skipif(torch.cuda.is_available(),
                             reason="made-up device addresses: host-only")


@_NO_GPU
def test_argument_errors_are_reported_before_any_launch():
    L = B.load()
    d = B.make_dims(128, 1)
    cc = _cache_c()
    ws = 0x10000
    by = ctypes.byref
    # null weight piece
    assert L.pack_quantize_weights(by(d), None, 96, ws, 96, ws, 128, by(cc), ws, 1 << 20, None) == 1
    # ld smaller than the piece width
    assert L.pack_quantize_weights(by(d), ws, 95, ws, 96, ws, 128, by(cc), ws, 1 << 20, None) == 1
    # misaligned piece and ld
    assert L.pack_quantize_weights(by(d), ws + 4, 96, ws, 96, ws, 128, by(cc), ws, 1 << 20, None) == 3
    assert L.pack_quantize_weights(by(d), ws, 98, ws, 96, ws, 128, by(cc), ws, 1 << 20, None) == 3
    # workspace too small
    assert L.pack_quantize_weights(by(d), ws, 96, ws, 96, ws, 128, by(cc), ws, 16, None) == 4
    # bad shapes
    bad = B.make_dims(100, 1)
    assert L.pack_quantize_weights(by(bad), ws, 96, ws, 96, ws, 128, by(cc), ws, 1 << 20, None) == 2
    # forward: non-positive sizes, null outputs, small saved buffer
    assert L.qkv_forward(by(d), 0, 256, ws, by(cc), ws, ws, ws, ws, 1 << 30, ws, 1 << 30, None) == 1
    assert L.qkv_forward(by(d), 1, 256, ws, by(cc), None, ws, ws, ws, 1 << 30, ws, 1 << 30, None) == 1
    assert L.qkv_forward(by(d), 1, 256, ws + 2, by(cc), ws, ws, ws, ws, 1 << 30, ws, 1 << 30, None) == 3
    assert L.qkv_forward(by(d), 1, 256, ws, by(cc), ws, ws, ws, ws, 10, ws, 1 << 30, None) == 4
    assert L.qkv_forward(by(d), 1 << 16, 1 << 15, ws, by(cc), ws, ws, ws, ws, 1 << 40, ws, 1 << 40,
                         None) == 2
    # forward with an incomplete weight cache
    half = B._CacheC(ws, None, ws, ws)
    assert L.qkv_forward(by(d), 1, 256, ws, by(half), ws, ws, ws, ws, 1 << 30, ws, 1 << 30, None) == 1
    # backward: ld errors on the dW outputs, missing or misaligned forward
    # outputs, small workspace
    assert L.qkv_backward(by(d), 1, 256, ws, ws, ws, ws, ws, ws, 1 << 30, by(cc), ws, ws, 90, ws,
                          96, ws, 128, ws, 1 << 30, None) == 1
    assert L.qkv_backward(by(d), 1, 256, None, ws, ws, ws, ws, ws, 1 << 30, by(cc), ws, ws, 96,
                          ws, 96, ws, 128, ws, 1 << 30, None) == 1
    assert L.qkv_backward(by(d), 1, 256, ws, ws + 8, ws, ws, ws, ws, 1 << 30, by(cc), ws, ws, 96,
                          ws, 96, ws, 128, ws, 1 << 30, None) == 3
    assert L.qkv_backward(by(d), 1, 256, ws, ws, ws, ws, ws, ws, 1 << 30, by(cc), ws, ws, 96, ws,
                          96, ws, 128, ws, 100, None) == 4
    # pack + forward in one call: the pack's and the forward's checks, and
    # a workspace that must hold both parts
    pf = B.workspace_bytes(d, 256, B.FPR_CALL_PACK_FORWARD)
    sv = B.saved_bytes(d, 256)
    args = [by(d), ws, 96, ws, 96, ws, 128, by(cc), 1, 256, ws, ws, ws, ws, ws, sv, ws, pf, None]

    def pack_fwd(**change):
        a = list(args)
        for i, val in change.items():
            a[int(i[1:])] = val
        return L.qkv_pack_forward(*a)

    assert pack_fwd(a1=None) == 1
    assert pack_fwd(a2=95) == 1
    assert pack_fwd(a8=0) == 1
    assert pack_fwd(a11=None) == 1
    assert pack_fwd(a10=ws + 2) == 3
    assert pack_fwd(a3=ws + 4) == 3
    assert pack_fwd(a15=sv - 1) == 4
    assert pack_fwd(a17=pf - 1) == 4
    assert pack_fwd(a17=B.workspace_bytes(d, 256, B.FPR_CALL_FORWARD)) == 4
    assert pack_fwd(a7=by(half)) == 1
    assert L.qkv_pack_forward(by(bad), *args[1:]) == 2
    # measurement hooks
    assert L.fpr_probe_copy(ws, ws + 8, 1024, 4, None) == 3
    assert L.fpr_probe_copy(ws, ws, 1000, 4, None) == 3
    assert L.fpr_probe_read(None, 1024, ws, 4, None) == 1
    assert L.fpr_probe_mfma(0, 10, ws, None) == -1
    # encoder hook
    assert L.fpr_e4m3_encode(ws, 15, 1.0, ws, None) == 3
    assert L.fpr_e4m3_encode(None, 16, 1.0, ws, None) == 1


# ------------------------------------------------------- FP8 ReLU^2 MLP

@pytest.mark.parametrize("dims,ok", [((768, 3072), True), ((128, 512), True), ((192, 320), True),
                                     ((100, 3072), False), ((768, 3000), False),
                                     ((0, 3072), False), ((768, 1 << 17), False)])
def test_mlp_shape_support(dims, ok):
    d = B.MlpDims(*dims)
    assert (B.mlp_saved_bytes(d, 256) > 0) == ok
    assert (B.mlp_workspace_bytes(d, 256, B.FPR_CALL_BACKWARD) > 0) == ok


def test_mlp_layout_is_disjoint_and_sized():
    d = B.MlpDims(768, 3072)
    T = 65536
    lay = B.mlp_layout(d, T)
    saved = [(lay.saved_x8, T * 768), (lay.saved_h8, T * 3072), (lay.saved_x_scales, 8),
             (lay.saved_h_scales, 8)]
    bwd = [(lay.bwd_dy8, T * 768), (lay.bwd_dy_scales, 8), (lay.bwd_dpre, 2 * T * 3072),
           (lay.bwd_dpre8, T * 3072), (lay.bwd_dpre_scales, 8),
           (lay.bwd_dw_part, lay.dw1_splits * 768 * 3072 * 4)]
    for regions, total in ((saved, B.mlp_saved_bytes(d, T)),
                           (bwd, B.mlp_workspace_bytes(d, T, B.FPR_CALL_BACKWARD))):
        regions = sorted(regions)
        for (a, n), (b, _) in zip(regions, regions[1:]):
            assert a + n <= b
        assert regions[-1][0] + regions[-1][1] <= total
    assert lay.fwd_h + 2 * T * 3072 <= B.mlp_workspace_bytes(d, T, B.FPR_CALL_FORWARD)
    assert lay.dw1_splits == lay.dw2_splits == 7
    # mlp_pack_forward's workspace: the two weights' amax partials, aligned,
    # then the forward's
    fw = B.mlp_workspace_bytes(d, T, B.FPR_CALL_FORWARD)
    pk = B.mlp_workspace_bytes(d, 0, B.FPR_CALL_PACK)
    pf = B.mlp_workspace_bytes(d, T, B.FPR_CALL_PACK_FORWARD)
    assert fw + 2 * pk <= pf < fw + 2 * pk + 256


@_NO_GPU
def test_mlp_argument_errors_are_reported_before_any_launch():
    L = B.load()
    d = B.MlpDims(128, 512)
    p = 0x10000
    cc = B._MlpCacheC(p, p, p, p, p, p)
    by = ctypes.byref
    assert L.mlp_pack_quantize_weights(by(d), None, 512, p, 128, by(cc), p, 1 << 20, None) == 1
    assert L.mlp_pack_quantize_weights(by(d), p, 500, p, 128, by(cc), p, 1 << 20, None) == 1
    assert L.mlp_pack_quantize_weights(by(d), p, 514, p, 128, by(cc), p, 1 << 20, None) == 3
    assert L.mlp_pack_quantize_weights(by(d), p, 512, p, 128, by(cc), p, 8, None) == 4
    bad = B.MlpDims(100, 512)
    assert L.mlp_forward(by(bad), 256, p, by(cc), p, p, 1 << 30, p, 1 << 30, None) == 2
    assert L.mlp_forward(by(d), 0, p, by(cc), p, p, 1 << 30, p, 1 << 30, None) == 1
    assert L.mlp_forward(by(d), (1 << 24) + 1, p, by(cc), p, p, 1 << 40, p, 1 << 40, None) == 2
    assert L.mlp_forward(by(d), 256, p, by(cc), None, p, 1 << 30, p, 1 << 30, None) == 1
    assert L.mlp_forward(by(d), 256, p + 2, by(cc), p, p, 1 << 30, p, 1 << 30, None) == 3
    assert L.mlp_forward(by(d), 256, p, by(cc), p, p, 16, p, 1 << 30, None) == 4
    half = B._MlpCacheC(p, p, None, p, p, p)
    assert L.mlp_forward(by(d), 256, p, by(half), p, p, 1 << 30, p, 1 << 30, None) == 1
    # pack + forward in one call: the checks of both, a workspace for both
    pf = B.mlp_workspace_bytes(d, 256, B.FPR_CALL_PACK_FORWARD)
    sv = B.mlp_saved_bytes(d, 256)
    args = [by(d), p, 512, p, 128, by(cc), 256, p, p, p, sv, p, pf, None]

    def pack_fwd(**change):
        a = list(args)
        for i, val in change.items():
            a[int(i[1:])] = val
        return L.mlp_pack_forward(*a)

    assert pack_fwd(a1=None) == 1
    assert pack_fwd(a4=127) == 1
    assert pack_fwd(a2=514) == 3
    assert pack_fwd(a6=0) == 1
    assert pack_fwd(a8=None) == 1
    assert pack_fwd(a7=p + 2) == 3
    assert pack_fwd(a10=sv - 1) == 4
    assert pack_fwd(a12=pf - 1) == 4
    assert pack_fwd(a12=B.mlp_workspace_bytes(d, 256, B.FPR_CALL_FORWARD)) == 4
    assert pack_fwd(a5=by(half)) == 1
    assert L.mlp_pack_forward(by(bad), *args[1:]) == 2
    assert L.mlp_backward(by(d), 256, p, p, 1 << 30, by(cc), p, p, 500, p, 128, p, 1 << 30,
                          None) == 1
    assert L.mlp_backward(by(d), 256, p, p, 1 << 30, by(cc), p, p, 512, p, 128, p, 64,
                          None) == 4


@pytest.mark.parametrize("passes,dqk,ok", [(0, 96, True), (1, 96, True), (2, 96, True),
                                           (2, 64, True), (2, 128, True), (2, 48, False),
                                           (2, 112, False), (1, 48, True), (3, 96, False),
                                           (-1, 96, False)])
def test_bwd_passes_support(passes, dqk, ok):
    """The two-pass backward exists for the quad-lane widths only."""
    d = B.make_dims(768, 6, d_qk=dqk, bwd_passes=passes)
    assert (B.workspace_bytes(d, 256, B.FPR_CALL_BACKWARD) > 0) == ok


def test_two_pass_backward_needs_no_dqk_buffer():
    """Without dQK in memory the backward workspace is dQK's bytes smaller,
    the layout reports no dQK, and nothing else moves in size."""
    T = 4096
    one, two = B.make_dims(768, 6), B.make_dims(768, 6, bwd_passes=2)
    nq2 = 2 * 6 * 96
    wb1 = B.workspace_bytes(one, T, B.FPR_CALL_BACKWARD)
    wb2 = B.workspace_bytes(two, T, B.FPR_CALL_BACKWARD)
    assert wb1 - wb2 >= T * nq2 * 2 and wb1 - wb2 < T * nq2 * 2 + 4096
    assert B.layout(two, T).bwd_dqkv == B.NOT_PRESENT
    assert B.layout(one, T).bwd_dqkv != B.NOT_PRESENT
    assert B.saved_bytes(one, T) == B.saved_bytes(two, T)
    for which in (B.FPR_CALL_PACK, B.FPR_CALL_FORWARD):
        assert B.workspace_bytes(one, T, which) == B.workspace_bytes(two, T, which)
