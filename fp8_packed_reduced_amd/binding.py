"""ctypes binding of libfpr.so (C interface in include/fpr.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  There
is no fallback: if the library is not built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfpr.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fpr.h")

FPR_CALL_PACK, FPR_CALL_FORWARD, FPR_CALL_BACKWARD, FPR_CALL_PACK_FORWARD = 0, 1, 2, 3
STATUS_W_NONFINITE, STATUS_X_NONFINITE, STATUS_G_NONFINITE, STATUS_H_NONFINITE = 1, 2, 4, 8
FORMAT_E4M3, FORMAT_E5M2 = 0, 1
NOT_PRESENT = ctypes.c_size_t(-1).value  # a layout offset of "(size_t)-1"


class FprError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} (code {code})")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("qk_stride", ctypes.c_int32), ("grad_format", ctypes.c_int32),
                ("bwd_passes", ctypes.c_int32)]

    @property
    def n_packed(self) -> int:
        return self.n_heads * (2 * self.d_qk + self.d_v)

    @property
    def qk_row(self) -> int:
        """Row stride of the q/k/dq/dk heads (d_qk unless padded)."""
        return self.qk_stride or self.d_qk

    @property
    def n_q(self) -> int:
        return self.n_heads * self.d_qk


class _CacheC(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p), ("w_packed_t", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("status", ctypes.c_void_p)]


TRACE_MAX = 4096


class _TraceC(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("capacity", ctypes.c_int),
                ("count", ctypes.c_int), ("only", ctypes.c_char_p),
                ("names", ctypes.c_char_p * TRACE_MAX)]


class Layout(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("tokens_padded", ctypes.c_int64),
                ("saved_x8", ctypes.c_size_t), ("saved_rho", ctypes.c_size_t),
                ("saved_x_scales", ctypes.c_size_t), ("fwd_qk_pre", ctypes.c_size_t),
                ("bwd_dqkv", ctypes.c_size_t), ("bwd_g_scales", ctypes.c_size_t),
                ("bwd_g8", ctypes.c_size_t),
                ("bwd_dw_part", ctypes.c_size_t), ("dw_splits", ctypes.c_int32),
                ("bwd_amax_partials", ctypes.c_int32),
                ("k_block", ctypes.c_int32), ("act_block_rows", ctypes.c_int32)]

    @property
    def fused_forward(self) -> bool:
        """Norm and RoPE run in the forward GEMM's epilogue (no pre-norm rows)."""
        return self.fwd_qk_pre == NOT_PRESENT


class MlpDims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("grad_format", ctypes.c_int32)]


class _MlpCacheC(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w1_t", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w2_t", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("status", ctypes.c_void_p)]


class MlpLayout(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("tokens_padded", ctypes.c_int64),
                ("saved_x8", ctypes.c_size_t), ("saved_h8", ctypes.c_size_t),
                ("saved_x_scales", ctypes.c_size_t), ("saved_h_scales", ctypes.c_size_t),
                ("fwd_h", ctypes.c_size_t), ("bwd_dy8", ctypes.c_size_t),
                ("bwd_dy_scales", ctypes.c_size_t), ("bwd_dpre", ctypes.c_size_t),
                ("bwd_dpre8", ctypes.c_size_t), ("bwd_dpre_scales", ctypes.c_size_t),
                ("bwd_dw_part", ctypes.c_size_t), ("dw1_splits", ctypes.c_int32),
                ("dw2_splits", ctypes.c_int32)]


_lib = None
_V, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


def load():
    """Load libfpr.so (built in-tree by fp8_packed_reduced_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m fp8_packed_reduced_amd.build`")
    L = ctypes.CDLL(LIB_PATH)  # torch is imported first, so HIP resolves to torch's runtime
    P = ctypes.POINTER
    L.fpr_workspace_bytes.restype = _SZ
    L.fpr_workspace_bytes.argtypes = [P(Dims), _I64, ctypes.c_int]
    L.fpr_saved_bytes.restype = _SZ
    L.fpr_saved_bytes.argtypes = [P(Dims), _I64]
    L.fpr_get_layout.restype = ctypes.c_int
    L.fpr_get_layout.argtypes = [P(Dims), _I64, P(Layout)]
    L.fpr_status_string.restype = ctypes.c_char_p
    L.fpr_status_string.argtypes = [ctypes.c_int]
    L.pack_quantize_weights.restype = ctypes.c_int
    L.pack_quantize_weights.argtypes = [P(Dims), _V, _I64, _V, _I64, _V, _I64, P(_CacheC),
                                        _V, _SZ, _V]
    L.qkv_forward.restype = ctypes.c_int
    L.qkv_forward.argtypes = [P(Dims), _I32, _I32, _V, P(_CacheC), _V, _V, _V, _V, _SZ, _V,
                              _SZ, _V]
    L.qkv_pack_forward.restype = ctypes.c_int
    L.qkv_pack_forward.argtypes = [P(Dims), _V, _I64, _V, _I64, _V, _I64, P(_CacheC), _I32, _I32,
                                   _V, _V, _V, _V, _V, _SZ, _V, _SZ, _V]
    L.qkv_forward_noalloc.restype = ctypes.c_int
    L.qkv_forward_noalloc.argtypes = [P(Dims), _I32, _I32, _V, P(_CacheC), _V, _V, _V, _V, _SZ,
                                      _V]
    L.fpr_noalloc_scratch_bytes.restype = _SZ
    L.fpr_noalloc_scratch_bytes.argtypes = []
    L.qkv_backward.restype = ctypes.c_int
    L.qkv_backward.argtypes = [P(Dims), _I32, _I32, _V, _V, _V, _V, _V, _V, _SZ, P(_CacheC),
                               _V, _V, _I64, _V, _I64, _V, _I64, _V, _SZ, _V]
    L.fpr_trace_set.restype = None
    L.fpr_trace_set.argtypes = [ctypes.POINTER(_TraceC)]
    L.fpr_e4m3_encode.restype = ctypes.c_int
    L.fpr_e4m3_encode.argtypes = [_V, _I64, ctypes.c_float, _V, _V]
    L.fpr_probe_copy.restype = ctypes.c_int
    L.fpr_probe_copy.argtypes = [_V, _V, _I64, ctypes.c_int, _V]
    L.fpr_probe_read.restype = ctypes.c_int
    L.fpr_probe_read.argtypes = [_V, _I64, _V, ctypes.c_int, _V]
    L.fpr_probe_mfma.restype = _I64
    L.fpr_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, _V, _V]
    L.fpr_e5m2_encode.restype = ctypes.c_int
    L.fpr_e5m2_encode.argtypes = [_V, _I64, ctypes.c_float, _V, _V]
    L.fpr_mlp_workspace_bytes.restype = _SZ
    L.fpr_mlp_workspace_bytes.argtypes = [P(MlpDims), _I64, ctypes.c_int]
    L.fpr_mlp_saved_bytes.restype = _SZ
    L.fpr_mlp_saved_bytes.argtypes = [P(MlpDims), _I64]
    L.fpr_mlp_get_layout.restype = ctypes.c_int
    L.fpr_mlp_get_layout.argtypes = [P(MlpDims), _I64, P(MlpLayout)]
    L.mlp_pack_quantize_weights.restype = ctypes.c_int
    L.mlp_pack_quantize_weights.argtypes = [P(MlpDims), _V, _I64, _V, _I64, P(_MlpCacheC), _V,
                                            _SZ, _V]
    L.mlp_forward.restype = ctypes.c_int
    L.mlp_forward.argtypes = [P(MlpDims), _I64, _V, P(_MlpCacheC), _V, _V, _SZ, _V, _SZ, _V]
    L.mlp_pack_forward.restype = ctypes.c_int
    L.mlp_pack_forward.argtypes = [P(MlpDims), _V, _I64, _V, _I64, P(_MlpCacheC), _I64, _V, _V,
                                   _V, _SZ, _V, _SZ, _V]
    L.mlp_backward.restype = ctypes.c_int
    L.mlp_backward.argtypes = [P(MlpDims), _I64, _V, _V, _SZ, P(_MlpCacheC), _V, _V, _I64, _V,
                               _I64, _V, _SZ, _V]
    _lib = L
    return L


def declared_functions() -> list[str]:
    """Names the public header declares with FPR_API."""
    text = open(HEADER).read()
    return re.findall(r"^FPR_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)


def status_string(code: int) -> str:
    return load().fpr_status_string(code).decode()


def make_dims(d_model: int, n_heads: int, d_qk: int = 96, d_v: int = 128,
              eps: float = 1e-6, rope_base: float = 10000.0, qk_stride: int = 0,
              grad_format: int = FORMAT_E4M3, bwd_passes: int = 0) -> Dims:
    """qk_stride > d_qk pads every q/k head row with zeros to that width;
    grad_format FORMAT_E5M2 quantises the backward's packed gradient to e5m2;
    bwd_passes 2 runs the backward in two passes that never write dQK."""
    return Dims(d_model, n_heads, d_qk, d_v, eps, rope_base, qk_stride, grad_format, bwd_passes)


def workspace_bytes(dims: Dims, tokens: int, which: int) -> int:
    return int(load().fpr_workspace_bytes(ctypes.byref(dims), tokens, which))


def saved_bytes(dims: Dims, tokens: int) -> int:
    return int(load().fpr_saved_bytes(ctypes.byref(dims), tokens))


def layout(dims: Dims, tokens: int) -> Layout:
    out = Layout()
    rc = load().fpr_get_layout(ctypes.byref(dims), tokens, ctypes.byref(out))
    if rc:
        raise FprError(rc, "fpr_get_layout")
    return out


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, shape, what: str):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda:
        raise ValueError(f"{what}: want {dtype} {tuple(shape)} on the GPU, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _need_rows(t: torch.Tensor, rows: int, cols: int, what: str) -> int:
    """2-D fp32 with unit column stride; returns its row stride."""
    if t.dtype != torch.float32 or t.dim() != 2 or tuple(t.shape) != (rows, cols) or not t.is_cuda:
        raise ValueError(f"{what}: want float32 ({rows}, {cols}) on the GPU")
    if t.stride(1) != 1:
        raise ValueError(f"{what} needs unit column stride")
    return t.stride(0)


class WeightCache:
    """Device buffers of the cached FP8 weight views (rebuilt per update)."""

    def __init__(self, dims: Dims, device="cuda"):
        D, N = dims.d_model, dims.n_packed
        self.dims = dims
        self.w_packed = torch.empty((D, N), dtype=torch.uint8, device=device)
        self.w_packed_t = torch.empty((N, D), dtype=torch.uint8, device=device)
        self.scales = torch.zeros(2, dtype=torch.float32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)

    def c(self) -> _CacheC:
        return _CacheC(self.w_packed.data_ptr(), self.w_packed_t.data_ptr(),
                       self.scales.data_ptr(), self.status.data_ptr())


def pack_quantize_weights(dims: Dims, wq, wk, wv, cache: WeightCache, workspace=None):
    D, nq, nv = dims.d_model, dims.n_q, dims.n_heads * dims.d_v
    ldq = _need_rows(wq, D, nq, "wq")
    ldk = _need_rows(wk, D, nq, "wk")
    ldv = _need_rows(wv, D, nv, "wv")
    dev = wq.device
    nbytes = workspace_bytes(dims, 0, FPR_CALL_PACK)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    cc = cache.c()
    rc = load().pack_quantize_weights(ctypes.byref(dims), wq.data_ptr(), ldq, wk.data_ptr(), ldk,
                                      wv.data_ptr(), ldv, ctypes.byref(cc), workspace.data_ptr(),
                                      workspace.numel(), _stream(dev))
    if rc:
        raise FprError(rc, "pack_quantize_weights")
    return cache


def qkv_forward(dims: Dims, n_seq: int, seq_len: int, x, cache: WeightCache, q=None, k=None,
                v=None, saved=None, workspace=None):
    """Returns (q, k, v, saved)."""
    T = n_seq * seq_len
    H, dqk, dv = dims.n_heads, dims.qk_row, dims.d_v
    dev = x.device
    _need(x, torch.bfloat16, (T, dims.d_model), "x")
    if q is None:
        q = torch.empty((n_seq, H, seq_len, dqk), dtype=torch.bfloat16, device=dev)
    if k is None:
        k = torch.empty((n_seq, H, seq_len, dqk), dtype=torch.bfloat16, device=dev)
    if v is None:
        v = torch.empty((n_seq, H, seq_len, dv), dtype=torch.bfloat16, device=dev)
    _need(q, torch.bfloat16, (n_seq, H, seq_len, dqk), "q")
    _need(k, torch.bfloat16, (n_seq, H, seq_len, dqk), "k")
    _need(v, torch.bfloat16, (n_seq, H, seq_len, dv), "v")
    if saved is None:
        saved = torch.empty(saved_bytes(dims, T), dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(dims, T, FPR_CALL_FORWARD), dtype=torch.uint8,
                                device=dev)
    cc = cache.c()
    rc = load().qkv_forward(ctypes.byref(dims), n_seq, seq_len, x.data_ptr(), ctypes.byref(cc),
                            q.data_ptr(), k.data_ptr(), v.data_ptr(), saved.data_ptr(),
                            saved.numel(), workspace.data_ptr(), workspace.numel(), _stream(dev))
    if rc:
        raise FprError(rc, "qkv_forward")
    return q, k, v, saved


def qkv_pack_forward(dims: Dims, wq, wk, wv, cache: WeightCache, n_seq: int, seq_len: int, x,
                     q=None, k=None, v=None, saved=None, workspace=None):
    """pack_quantize_weights then qkv_forward in one call (shared launches).
    Returns (q, k, v, saved)."""
    T = n_seq * seq_len
    D, nq, nv = dims.d_model, dims.n_q, dims.n_heads * dims.d_v
    H, dqk, dv = dims.n_heads, dims.qk_row, dims.d_v
    ldq = _need_rows(wq, D, nq, "wq")
    ldk = _need_rows(wk, D, nq, "wk")
    ldv = _need_rows(wv, D, nv, "wv")
    dev = x.device
    _need(x, torch.bfloat16, (T, D), "x")
    if q is None:
        q = torch.empty((n_seq, H, seq_len, dqk), dtype=torch.bfloat16, device=dev)
    if k is None:
        k = torch.empty((n_seq, H, seq_len, dqk), dtype=torch.bfloat16, device=dev)
    if v is None:
        v = torch.empty((n_seq, H, seq_len, dv), dtype=torch.bfloat16, device=dev)
    _need(q, torch.bfloat16, (n_seq, H, seq_len, dqk), "q")
    _need(k, torch.bfloat16, (n_seq, H, seq_len, dqk), "k")
    _need(v, torch.bfloat16, (n_seq, H, seq_len, dv), "v")
    if saved is None:
        saved = torch.empty(saved_bytes(dims, T), dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(dims, T, FPR_CALL_PACK_FORWARD),
                                dtype=torch.uint8, device=dev)
    cc = cache.c()
    rc = load().qkv_pack_forward(ctypes.byref(dims), wq.data_ptr(), ldq, wk.data_ptr(), ldk,
                                 wv.data_ptr(), ldv, ctypes.byref(cc), n_seq, seq_len,
                                 x.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 saved.data_ptr(), saved.numel(), workspace.data_ptr(),
                                 workspace.numel(), _stream(dev))
    if rc:
        raise FprError(rc, "qkv_pack_forward")
    return q, k, v, saved


def qkv_forward_noalloc(dims: Dims, n_seq: int, seq_len: int, x, cache: WeightCache, q, k, v,
                        saved):
    """qkv_forward with its workspace in the library's fixed per-device
    scratch: the caller passes only inputs and outputs (all preallocated)."""
    T = n_seq * seq_len
    H, dqk, dv = dims.n_heads, dims.qk_row, dims.d_v
    _need(x, torch.bfloat16, (T, dims.d_model), "x")
    _need(q, torch.bfloat16, (n_seq, H, seq_len, dqk), "q")
    _need(k, torch.bfloat16, (n_seq, H, seq_len, dqk), "k")
    _need(v, torch.bfloat16, (n_seq, H, seq_len, dv), "v")
    cc = cache.c()
    rc = load().qkv_forward_noalloc(ctypes.byref(dims), n_seq, seq_len, x.data_ptr(),
                                    ctypes.byref(cc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    saved.data_ptr(), saved.numel(), _stream(x.device))
    if rc:
        raise FprError(rc, "qkv_forward_noalloc")
    return q, k, v, saved


def noalloc_scratch_bytes() -> int:
    return int(load().fpr_noalloc_scratch_bytes())


def qkv_backward(dims: Dims, n_seq: int, seq_len: int, q, k, dq, dk, dv, saved,
                 cache: WeightCache, dx=None, dw=None, workspace=None):
    """q, k: the matching forward's outputs.  Returns (dx, dw) with dw the
    [D][N] packed fp32 gradient whose column blocks [:nq], [nq:2nq], [2nq:]
    are dW_q, dW_k, dW_v."""
    T = n_seq * seq_len
    H, dqk, dvw, D, N, nq = dims.n_heads, dims.qk_row, dims.d_v, dims.d_model, dims.n_packed, dims.n_q
    dev = dq.device
    _need(q, torch.bfloat16, (n_seq, H, seq_len, dqk), "q")
    _need(k, torch.bfloat16, (n_seq, H, seq_len, dqk), "k")
    _need(dq, torch.bfloat16, (n_seq, H, seq_len, dqk), "dq")
    _need(dk, torch.bfloat16, (n_seq, H, seq_len, dqk), "dk")
    _need(dv, torch.bfloat16, (n_seq, H, seq_len, dvw), "dv")
    if dx is None:
        dx = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    _need(dx, torch.bfloat16, (T, D), "dx")
    if dw is None:
        dw = torch.empty((D, N), dtype=torch.float32, device=dev)
    _need(dw, torch.float32, (D, N), "dw")
    if workspace is None:
        workspace = torch.empty(workspace_bytes(dims, T, FPR_CALL_BACKWARD), dtype=torch.uint8,
                                device=dev)
    dwq, dwk, dwv = dw[:, :nq], dw[:, nq:2 * nq], dw[:, 2 * nq:]
    cc = cache.c()
    rc = load().qkv_backward(ctypes.byref(dims), n_seq, seq_len, q.data_ptr(), k.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), saved.data_ptr(),
                             saved.numel(), ctypes.byref(cc),
                             dx.data_ptr(), dwq.data_ptr(), N, dwk.data_ptr(), N, dwv.data_ptr(),
                             N, workspace.data_ptr(), workspace.numel(), _stream(dev))
    if rc:
        raise FprError(rc, "qkv_backward")
    return dx, dw


def e4m3_encode(values: torch.Tensor, inv_scale: float = 1.0, e5m2: bool = False) -> torch.Tensor:
    """Device encoder hook: e4m3(values * inv_scale) (or e5m2), no amax."""
    if values.dtype != torch.float32 or not values.is_cuda or not values.is_contiguous():
        raise ValueError("values must be a contiguous float32 GPU tensor")
    out = torch.empty(values.shape, dtype=torch.uint8, device=values.device)
    fn, name = ((load().fpr_e5m2_encode, "fpr_e5m2_encode") if e5m2
                else (load().fpr_e4m3_encode, "fpr_e4m3_encode"))
    rc = fn(values.data_ptr(), values.numel(), inv_scale, out.data_ptr(), _stream(values.device))
    if rc:
        raise FprError(rc, name)
    return out


def probe_copy(src: torch.Tensor, dst: torch.Tensor, blocks: int):
    """Measurement hook: streaming copy of src's bytes into dst."""
    rc = load().fpr_probe_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(),
                               blocks, _stream(src.device))
    if rc:
        raise FprError(rc, "fpr_probe_copy")


def probe_read(src: torch.Tensor, out: torch.Tensor, blocks: int):
    """Measurement hook: streaming read of src's bytes (one word per block to out)."""
    rc = load().fpr_probe_read(src.data_ptr(), src.numel() * src.element_size(), out.data_ptr(),
                               blocks, _stream(src.device))
    if rc:
        raise FprError(rc, "fpr_probe_read")


def probe_mfma(blocks: int, iters: int, out: torch.Tensor) -> int:
    """Measurement hook: the bare FP8 MFMA loop; returns the FLOP it does."""
    flop = load().fpr_probe_mfma(blocks, iters, out.data_ptr(), _stream(out.device))
    if flop < 0:
        raise FprError(-flop, "fpr_probe_mfma")
    return int(flop)


def view_bytes(buf: torch.Tensor, offset: int, shape, dtype) -> torch.Tensor:
    """A typed view into a byte buffer (for reading intermediates in tests)."""
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return buf[offset:offset + nbytes].view(dtype).view(*shape)


class KernelTrace:
    """Brackets the library's kernels with torch (HIP) timing events on the
    launch stream.  Use as a context manager around calls made on this
    thread; ``only`` restricts it to one stage name."""

    def __init__(self, capacity: int, only: str | None = None, device=None):
        capacity = min(capacity, TRACE_MAX)
        stream = torch.cuda.current_stream(device)
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * capacity)]
        for e in self.events:       # materialise the underlying hipEvent_t
            e.record(stream)
        torch.cuda.synchronize(device)
        self._handles = (ctypes.c_void_p * (2 * capacity))(*[e.cuda_event for e in self.events])
        self._only = only.encode() if only else None
        self._c = _TraceC(ctypes.cast(self._handles, ctypes.POINTER(ctypes.c_void_p)), capacity,
                          0, self._only)

    def __enter__(self):
        load().fpr_trace_set(ctypes.byref(self._c))
        return self

    def __exit__(self, *exc):
        load().fpr_trace_set(None)
        return False

    def records(self):
        """[(stage name, milliseconds)] in launch order (call after a sync)."""
        out = []
        for i in range(self._c.count):
            name = self._c.names[i].decode()
            out.append((name, self.events[2 * i].elapsed_time(self.events[2 * i + 1])))
        return out


# ------------------------------------------------------- FP8 ReLU^2 MLP

def mlp_workspace_bytes(dims: MlpDims, tokens: int, which: int) -> int:
    return int(load().fpr_mlp_workspace_bytes(ctypes.byref(dims), tokens, which))


def mlp_saved_bytes(dims: MlpDims, tokens: int) -> int:
    return int(load().fpr_mlp_saved_bytes(ctypes.byref(dims), tokens))


def mlp_layout(dims: MlpDims, tokens: int) -> MlpLayout:
    out = MlpLayout()
    rc = load().fpr_mlp_get_layout(ctypes.byref(dims), tokens, ctypes.byref(out))
    if rc:
        raise FprError(rc, "fpr_mlp_get_layout")
    return out


class MlpCache:
    """Device buffers of the cached FP8 views of W1 and W2."""

    def __init__(self, dims: MlpDims, device="cuda"):
        D, F = dims.d_model, dims.d_ff
        self.dims = dims
        self.w1 = torch.empty((D, F), dtype=torch.uint8, device=device)
        self.w1_t = torch.empty((F, D), dtype=torch.uint8, device=device)
        self.w2 = torch.empty((F, D), dtype=torch.uint8, device=device)
        self.w2_t = torch.empty((D, F), dtype=torch.uint8, device=device)
        self.scales = torch.zeros(4, dtype=torch.float32, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)

    def c(self) -> _MlpCacheC:
        return _MlpCacheC(self.w1.data_ptr(), self.w1_t.data_ptr(), self.w2.data_ptr(),
                          self.w2_t.data_ptr(), self.scales.data_ptr(), self.status.data_ptr())


def mlp_pack_quantize_weights(dims: MlpDims, w1, w2, cache: MlpCache, workspace=None):
    D, F = dims.d_model, dims.d_ff
    ld1 = _need_rows(w1, D, F, "w1")
    ld2 = _need_rows(w2, F, D, "w2")
    if workspace is None:
        workspace = torch.empty(mlp_workspace_bytes(dims, 0, FPR_CALL_PACK), dtype=torch.uint8,
                                device=w1.device)
    cc = cache.c()
    rc = load().mlp_pack_quantize_weights(ctypes.byref(dims), w1.data_ptr(), ld1, w2.data_ptr(),
                                          ld2, ctypes.byref(cc), workspace.data_ptr(),
                                          workspace.numel(), _stream(w1.device))
    if rc:
        raise FprError(rc, "mlp_pack_quantize_weights")
    return cache


def mlp_forward(dims: MlpDims, x, cache: MlpCache, y=None, saved=None, workspace=None):
    """Returns (y, saved)."""
    T, D = x.shape[0], dims.d_model
    dev = x.device
    _need(x, torch.bfloat16, (T, D), "x")
    if y is None:
        y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    _need(y, torch.bfloat16, (T, D), "y")
    if saved is None:
        saved = torch.empty(mlp_saved_bytes(dims, T), dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = torch.empty(mlp_workspace_bytes(dims, T, FPR_CALL_FORWARD),
                                dtype=torch.uint8, device=dev)
    cc = cache.c()
    rc = load().mlp_forward(ctypes.byref(dims), T, x.data_ptr(), ctypes.byref(cc), y.data_ptr(),
                            saved.data_ptr(), saved.numel(), workspace.data_ptr(),
                            workspace.numel(), _stream(dev))
    if rc:
        raise FprError(rc, "mlp_forward")
    return y, saved


def mlp_pack_forward(dims: MlpDims, w1, w2, cache: MlpCache, x, y=None, saved=None,
                     workspace=None):
    """mlp_pack_quantize_weights then mlp_forward in one call (shared
    launches).  Returns (y, saved)."""
    T, D, F = x.shape[0], dims.d_model, dims.d_ff
    ld1 = _need_rows(w1, D, F, "w1")
    ld2 = _need_rows(w2, F, D, "w2")
    dev = x.device
    _need(x, torch.bfloat16, (T, D), "x")
    if y is None:
        y = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    _need(y, torch.bfloat16, (T, D), "y")
    if saved is None:
        saved = torch.empty(mlp_saved_bytes(dims, T), dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = torch.empty(mlp_workspace_bytes(dims, T, FPR_CALL_PACK_FORWARD),
                                dtype=torch.uint8, device=dev)
    cc = cache.c()
    rc = load().mlp_pack_forward(ctypes.byref(dims), w1.data_ptr(), ld1, w2.data_ptr(), ld2,
                                 ctypes.byref(cc), T, x.data_ptr(), y.data_ptr(),
                                 saved.data_ptr(), saved.numel(), workspace.data_ptr(),
                                 workspace.numel(), _stream(dev))
    if rc:
        raise FprError(rc, "mlp_pack_forward")
    return y, saved


def mlp_backward(dims: MlpDims, dy, saved, cache: MlpCache, dx=None, dw1=None, dw2=None,
                 workspace=None):
    """Returns (dx, dw1, dw2)."""
    T, D, F = dy.shape[0], dims.d_model, dims.d_ff
    dev = dy.device
    _need(dy, torch.bfloat16, (T, D), "dy")
    if dx is None:
        dx = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    _need(dx, torch.bfloat16, (T, D), "dx")
    if dw1 is None:
        dw1 = torch.empty((D, F), dtype=torch.float32, device=dev)
    if dw2 is None:
        dw2 = torch.empty((F, D), dtype=torch.float32, device=dev)
    ld1 = _need_rows(dw1, D, F, "dw1")
    ld2 = _need_rows(dw2, F, D, "dw2")
    if workspace is None:
        workspace = torch.empty(mlp_workspace_bytes(dims, T, FPR_CALL_BACKWARD),
                                dtype=torch.uint8, device=dev)
    cc = cache.c()
    rc = load().mlp_backward(ctypes.byref(dims), T, dy.data_ptr(), saved.data_ptr(),
                             saved.numel(), ctypes.byref(cc), dx.data_ptr(), dw1.data_ptr(), ld1,
                             dw2.data_ptr(), ld2, workspace.data_ptr(), workspace.numel(),
                             _stream(dev))
    if rc:
        raise FprError(rc, "mlp_backward")
    return dx, dw1, dw2
