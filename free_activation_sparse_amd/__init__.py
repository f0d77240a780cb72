"""Python binding of the weight-informed activation-sparse linear (C ABI in
include/sparse_linear.h) and of Double Sparsity decode attention (C ABI in
include/double_sparse.h); HIP kernels for gfx950 in csrc/.

Argument marshalling only: every step of the forward runs in the library's
kernels. PyTorch supplies device memory and streams. Loading fails loudly when
the built library is missing; there is no fallback path.

The functions below carry the C names; ``SparseLinear`` wraps a handle for
torch tensors; ``label_cache_update`` and ``decode_attention`` take torch
tensors for the Double Sparsity calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_linear.so")

SL_OK, SL_ERR_ARG, SL_ERR_UNSUPPORTED, SL_ERR_OOM, SL_ERR_HIP = 0, 1, 2, 3, 4
SL_F32, SL_BF16 = 0, 1
SL_W_ROWMAJOR_OUT_IN, SL_W_COLMAJOR = 0, 1
SL_GATE_TOPK, SL_GATE_STAT, SL_GATE_FIXED = 0, 1, 2
SL_MAX_N, SL_MAX_BATCH = 32768, 16
SL_STAGE_GATE, SL_STAGE_PRODUCT = 1, 2
DS_MAX_SEQ, DS_MAX_K = 32768, 8192

EXPORTED = [
    "sparse_linear_init", "sparse_linear_forward", "sparse_linear_forward_dense",
    "sparse_linear_get_norms", "sparse_linear_destroy", "sparse_linear_strerror",
    "sparse_linear_last_error", "sparse_linear_normal_quantile",
    "sparse_linear_forward_stages", "sparse_linear_set_plan", "sparse_linear_set_deterministic",
    "sparse_linear_set_union_plan", "sparse_linear_set_fused", "sparse_linear_sync_status",
    "sparse_linear_forward_group", "sparse_linear_forward_group_batch", "sparse_linear_ffn_workspace_bytes", "sparse_linear_forward_ffn",
    "sparse_linear_forward_ffn_noalloc",
    "sparse_linear_gather_ceiling", "sparse_linear_set_timeline", "ds_label_cache_update", "ds_decode_attention",
]

_lib: Optional[ctypes.CDLL] = None

_vp, _i64, _i32, _dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double


class SparseLinearError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run python -m free_activation_sparse_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    L.sparse_linear_init.argtypes = [ctypes.POINTER(_vp), _vp, ctypes.c_int, ctypes.c_int, _i64, _i64, _vp,
                                     ctypes.c_int, _i64, _dbl, _i32, _vp]
    L.sparse_linear_init.restype = ctypes.c_int
    L.sparse_linear_forward.argtypes = [_vp, _vp, _i32, _vp, ctypes.c_int, _vp, _vp, _vp, _vp]
    L.sparse_linear_forward.restype = ctypes.c_int
    L.sparse_linear_forward_dense.argtypes = [_vp, _vp, _i32, _vp, ctypes.c_int, _vp]
    L.sparse_linear_forward_dense.restype = ctypes.c_int
    L.sparse_linear_forward_group.argtypes = [_vp, _i32, _vp, _vp, ctypes.c_int, _vp]
    L.sparse_linear_forward_group.restype = ctypes.c_int
    L.sparse_linear_forward_group_batch.argtypes = [_vp, _i32, _vp, _i32, _vp, ctypes.c_int, _vp]
    L.sparse_linear_forward_group_batch.restype = ctypes.c_int
    L.sparse_linear_ffn_workspace_bytes.argtypes = [_vp]
    L.sparse_linear_ffn_workspace_bytes.restype = _i64
    L.sparse_linear_forward_ffn.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _i64, _vp]
    L.sparse_linear_forward_ffn.restype = ctypes.c_int
    L.sparse_linear_forward_ffn_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp]
    L.sparse_linear_forward_ffn_noalloc.restype = ctypes.c_int
    L.sparse_linear_get_norms.argtypes = [_vp, _vp, _vp]
    L.sparse_linear_get_norms.restype = ctypes.c_int
    L.sparse_linear_destroy.argtypes = [_vp]
    L.sparse_linear_destroy.restype = ctypes.c_int
    L.sparse_linear_strerror.argtypes = [ctypes.c_int]
    L.sparse_linear_strerror.restype = ctypes.c_char_p
    L.sparse_linear_last_error.argtypes = []
    L.sparse_linear_last_error.restype = ctypes.c_char_p
    L.sparse_linear_normal_quantile.argtypes = [_dbl]
    L.sparse_linear_normal_quantile.restype = _dbl
    L.sparse_linear_forward_stages.argtypes = [_vp, _vp, _i32, _vp, ctypes.c_int, _vp, _vp, _vp, _i32, _vp]
    L.sparse_linear_forward_stages.restype = ctypes.c_int
    L.sparse_linear_set_deterministic.argtypes = [_vp, _i32]
    L.sparse_linear_set_deterministic.restype = ctypes.c_int
    L.sparse_linear_set_union_plan.argtypes = [_vp, _i32, _i32]
    L.sparse_linear_set_union_plan.restype = ctypes.c_int
    L.sparse_linear_set_plan.argtypes = [_vp, _i32, _i32]
    L.sparse_linear_set_plan.restype = ctypes.c_int
    L.sparse_linear_set_fused.argtypes = [_vp, _i32]
    L.sparse_linear_set_fused.restype = ctypes.c_int
    L.sparse_linear_sync_status.argtypes = [_vp, _vp]
    L.sparse_linear_sync_status.restype = ctypes.c_int
    L.sparse_linear_gather_ceiling.argtypes = [_vp, _vp, _i32, _vp, _vp]
    L.sparse_linear_gather_ceiling.restype = ctypes.c_int
    L.sparse_linear_set_timeline.argtypes = [_vp]
    L.sparse_linear_set_timeline.restype = ctypes.c_int
    L.ds_label_cache_update.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]
    L.ds_label_cache_update.restype = ctypes.c_int
    L.ds_decode_attention.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                      ctypes.c_float, _vp, _vp, _vp]
    L.ds_decode_attention.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != SL_OK:
        msg = lib().sparse_linear_last_error().decode(errors="replace")
        raise SparseLinearError(status, where, msg or lib().sparse_linear_strerror(status).decode())


# ------------------------------------------------------------------ C names
def sparse_linear_init(W_ptr: int, w_dtype: int, w_layout: int, m: int, n: int, c_ptr: int, gate: int,
                       K: int, s_keep: float, max_batch: int, stream: int) -> int:
    h = _vp()
    _check(lib().sparse_linear_init(ctypes.byref(h), W_ptr, w_dtype, w_layout, m, n, c_ptr or None, gate,
                                    K, s_keep, max_batch, stream or None), "sparse_linear_init")
    return h.value


def sparse_linear_forward(h: int, x_ptr: int, B: int, y_ptr: int, y_dtype: int, mask_ptr: int = 0,
                          count_ptr: int = 0, thresh_ptr: int = 0, stream: int = 0) -> None:
    _check(lib().sparse_linear_forward(h, x_ptr, B, y_ptr, y_dtype, mask_ptr or None, count_ptr or None,
                                       thresh_ptr or None, stream or None), "sparse_linear_forward")


def sparse_linear_forward_group(handles, x_ptr: int, y_ptrs, y_dtype: int, stream: int = 0) -> None:
    """One token through len(handles) linears that share x (handles and
    y_ptrs: sequences of ints)."""
    count = len(handles)
    ha = (_vp * max(1, count))(*handles)
    ya = (_vp * max(1, count))(*y_ptrs)
    _check(lib().sparse_linear_forward_group(ha, count, x_ptr, ya, y_dtype, stream or None),
           "sparse_linear_forward_group")


def sparse_linear_forward_group_batch(handles, x_ptr: int, B: int, y_ptrs, y_dtype: int, stream: int = 0) -> None:
    """B tokens ([B][n]) through len(handles) linears that share x."""
    count = len(handles)
    ha = (_vp * max(1, count))(*handles)
    ya = (_vp * max(1, count))(*y_ptrs)
    _check(lib().sparse_linear_forward_group_batch(ha, count, x_ptr, B, ya, y_dtype, stream or None),
           "sparse_linear_forward_group_batch")


def sparse_linear_ffn_workspace_bytes(up: int) -> int:
    return int(lib().sparse_linear_ffn_workspace_bytes(up))


def sparse_linear_forward_ffn(gate: int, up: int, down: int, x_ptr: int, y_ptr: int, y_dtype: int, ws_ptr: int,
                              ws_bytes: int, stream: int = 0) -> None:
    _check(lib().sparse_linear_forward_ffn(gate, up, down, x_ptr, y_ptr, y_dtype, ws_ptr, ws_bytes, stream or None),
           "sparse_linear_forward_ffn")


def sparse_linear_forward_ffn_noalloc(gate: int, up: int, down: int, x_ptr: int, y_ptr: int, y_dtype: int,
                                      stream: int = 0) -> None:
    _check(lib().sparse_linear_forward_ffn_noalloc(gate, up, down, x_ptr, y_ptr, y_dtype, stream or None),
           "sparse_linear_forward_ffn_noalloc")


def ds_label_cache_update(key_ptr: int, label_ptr: int, channels_ptr: int, start_ptr: int, batch: int, heads: int,
                          max_seq: int, head_dim: int, r: int, span: int, stream: int = 0) -> None:
    _check(lib().ds_label_cache_update(key_ptr, label_ptr, channels_ptr, start_ptr or None, batch, heads, max_seq,
                                       head_dim, r, span, stream or None), "ds_label_cache_update")


def ds_decode_attention(q_ptr: int, key_ptr: int, value_ptr: int, label_ptr: int, channels_ptr: int,
                        seq_len_ptr: int, batch: int, heads: int, max_seq: int, head_dim: int, r: int, k: int,
                        scale: float, out_ptr: int, tokens_out_ptr: int = 0, stream: int = 0) -> None:
    _check(lib().ds_decode_attention(q_ptr, key_ptr, value_ptr, label_ptr or None, channels_ptr, seq_len_ptr,
                                     batch, heads, max_seq, head_dim, r, k, scale, out_ptr,
                                     tokens_out_ptr or None, stream or None), "ds_decode_attention")


def sparse_linear_forward_dense(h: int, x_ptr: int, B: int, y_ptr: int, y_dtype: int, stream: int = 0) -> None:
    _check(lib().sparse_linear_forward_dense(h, x_ptr, B, y_ptr, y_dtype, stream or None),
           "sparse_linear_forward_dense")


def sparse_linear_get_norms(h: int, c_ptr: int, stream: int = 0) -> None:
    _check(lib().sparse_linear_get_norms(h, c_ptr, stream or None), "sparse_linear_get_norms")


def sparse_linear_destroy(h: int) -> None:
    _check(lib().sparse_linear_destroy(h), "sparse_linear_destroy")


def sparse_linear_strerror(status: int) -> str:
    return lib().sparse_linear_strerror(status).decode()


def sparse_linear_last_error() -> str:
    return lib().sparse_linear_last_error().decode(errors="replace")


def sparse_linear_normal_quantile(p: float) -> float:
    return lib().sparse_linear_normal_quantile(p)


def sparse_linear_forward_stages(h: int, x_ptr: int, B: int, y_ptr: int, y_dtype: int, mask_ptr: int = 0,
                                 count_ptr: int = 0, thresh_ptr: int = 0, stages: int = 3,
                                 stream: int = 0) -> None:
    _check(lib().sparse_linear_forward_stages(h, x_ptr, B, y_ptr, y_dtype, mask_ptr or None, count_ptr or None,
                                              thresh_ptr or None, stages, stream or None),
           "sparse_linear_forward_stages")


def sparse_linear_gather_ceiling(h: int, idx_ptr: int, count: int, sink_ptr: int, stream: int = 0) -> None:
    _check(lib().sparse_linear_gather_ceiling(h, idx_ptr, count, sink_ptr, stream or None),
           "sparse_linear_gather_ceiling")


def sparse_linear_set_timeline(buf_ptr: int) -> None:
    _check(lib().sparse_linear_set_timeline(buf_ptr or None), "sparse_linear_set_timeline")


def sparse_linear_set_deterministic(h: int, on: bool) -> None:
    _check(lib().sparse_linear_set_deterministic(h, 1 if on else 0), "sparse_linear_set_deterministic")


def sparse_linear_set_union_plan(h: int, rows_per_tile: int, workgroups: int) -> None:
    _check(lib().sparse_linear_set_union_plan(h, rows_per_tile, workgroups), "sparse_linear_set_union_plan")


def sparse_linear_set_plan(h: int, rows_per_tile: int, splits: int) -> None:
    _check(lib().sparse_linear_set_plan(h, rows_per_tile, splits), "sparse_linear_set_plan")


def sparse_linear_set_fused(h: int, on: bool) -> None:
    _check(lib().sparse_linear_set_fused(h, 1 if on else 0), "sparse_linear_set_fused")


def sparse_linear_sync_status(h: int, stream: int = 0) -> None:
    _check(lib().sparse_linear_sync_status(h, stream), "sparse_linear_sync_status")


# ------------------------------------------------------------------ torch wrapper
class SparseLinear:
    """One linear layer behind a library handle.

    ``W`` is a CUDA tensor [m][n] (nn.Linear layout) or, with
    ``layout='colmajor'``, the column-major [n][m] tensor; bf16 or fp32.
    ``gate`` is 'topk' (with K), 'stat' (with s_keep) or 'fixed' (with tau).
    """

    def __init__(self, W, c=None, gate: str = "topk", K: int = 0, s_keep: float = 0.0,
                 tau: float = 0.0, max_batch: int = 1, layout: str = "rowmajor", m: int = None,
                 n: int = None):
        import torch
        if not W.is_cuda:
            raise ValueError("W must be a device tensor")
        self._torch = torch
        self.dtype = W.dtype
        self.w_dtype = {torch.bfloat16: SL_BF16, torch.float32: SL_F32}[W.dtype]
        if layout == "rowmajor":
            m, n = W.shape
            lay = SL_W_ROWMAJOR_OUT_IN
        else:
            n, m = W.shape
            lay = SL_W_COLMAJOR
        W = W.contiguous()
        cp = 0
        if c is not None:
            c = c.to(device=W.device, dtype=torch.float32).contiguous()
            cp = c.data_ptr()
        g = {"topk": SL_GATE_TOPK, "stat": SL_GATE_STAT, "fixed": SL_GATE_FIXED}[gate]
        param = s_keep if g == SL_GATE_STAT else (tau if g == SL_GATE_FIXED else 0.0)
        self.m, self.n, self.max_batch, self.device = m, n, max_batch, W.device
        self.handle = sparse_linear_init(W.data_ptr(), self.w_dtype, lay, m, n, cp, g, K, param,
                                         max_batch, torch.cuda.current_stream(W.device).cuda_stream)

    def _stream(self):
        return self._torch.cuda.current_stream(self.device).cuda_stream

    def _out(self, B, y, y_dtype):
        torch = self._torch
        if y is None:
            y = torch.empty((B, self.m), dtype=y_dtype, device=self.device)
        return y

    def forward(self, x, y=None, y_dtype=None, mask: bool = False, count: bool = False,
                thresh: bool = False):
        torch = self._torch
        if x.dtype != self.dtype or not x.is_cuda or not x.is_contiguous():
            raise ValueError("x must be a contiguous device tensor of W's dtype")
        B = 1 if x.dim() == 1 else x.shape[0]
        y_dtype = torch.float32 if y_dtype is None else y_dtype
        y = self._out(B, y, y_dtype)
        mk = torch.empty((B, self.n), dtype=torch.uint8, device=self.device) if mask else None
        ct = torch.empty((B,), dtype=torch.int32, device=self.device) if count else None
        th = torch.empty((B,), dtype=torch.float64, device=self.device) if thresh else None
        sparse_linear_forward(self.handle, x.data_ptr(), B, y.data_ptr(),
                              SL_BF16 if y.dtype == torch.bfloat16 else SL_F32,
                              mk.data_ptr() if mk is not None else 0,
                              ct.data_ptr() if ct is not None else 0,
                              th.data_ptr() if th is not None else 0, self._stream())
        return {"y": y, "mask": mk, "count": ct, "thresh": th}

    @staticmethod
    def forward_group(layers, x, ys=None, y_dtype=None):
        """y_l = layers[l](x) for x shared by every layer (same n and dtype):
        one token ([n]) in one launch where possible, or B tokens ([B][n])
        with every layer's gates in one launch; returns the list of y ([m] or
        [B][m])."""
        torch = layers[0]._torch
        y_dtype = torch.float32 if y_dtype is None else y_dtype
        lead = tuple(x.shape[:-1]) if x.dim() > 1 else ()
        B = x.shape[0] if x.dim() > 1 else 1
        if ys is None:
            ys = [torch.empty(lead + (l.m,), dtype=y_dtype, device=l.device) for l in layers]
        ydt = SL_BF16 if ys[0].dtype == torch.bfloat16 else SL_F32
        if x.dim() > 1:
            sparse_linear_forward_group_batch([l.handle for l in layers], x.data_ptr(), B,
                                              [y.data_ptr() for y in ys], ydt, layers[0]._stream())
        else:
            sparse_linear_forward_group([l.handle for l in layers], x.data_ptr(), [y.data_ptr() for y in ys], ydt,
                                        layers[0]._stream())
        return ys

    @staticmethod
    def forward_ffn(gate, up, down, x, y=None, y_dtype=None, workspace=None):
        """y = down(bf16(SiLU(gate(x)) * up(x))) for one token, every step on
        the device. Returns (y, workspace); the workspace holds g, u (fp32)
        and h (bf16) at byte offsets 0, P and 2P, P = 256-aligned 4 * m."""
        torch = up._torch
        nb = sparse_linear_ffn_workspace_bytes(up.handle)
        if workspace is None:
            workspace = torch.empty((nb,), dtype=torch.uint8, device=up.device)
        y_dtype = torch.float32 if y_dtype is None else y_dtype
        if y is None:
            y = torch.empty((down.m,), dtype=y_dtype, device=down.device)
        sparse_linear_forward_ffn(gate.handle, up.handle, down.handle, x.data_ptr(), y.data_ptr(),
                                  SL_BF16 if y.dtype == torch.bfloat16 else SL_F32, workspace.data_ptr(),
                                  workspace.numel(), up._stream())
        return y, workspace

    def forward_dense(self, x, y=None, y_dtype=None):
        torch = self._torch
        B = 1 if x.dim() == 1 else x.shape[0]
        y_dtype = torch.float32 if y_dtype is None else y_dtype
        y = self._out(B, y, y_dtype)
        sparse_linear_forward_dense(self.handle, x.data_ptr(), B, y.data_ptr(),
                                    SL_BF16 if y.dtype == torch.bfloat16 else SL_F32, self._stream())
        return y

    def norms(self):
        c = self._torch.empty((self.n,), dtype=self._torch.float32, device=self.device)
        sparse_linear_get_norms(self.handle, c.data_ptr(), self._stream())
        return c

    def set_plan(self, rows_per_tile: int = 0, splits: int = 0):
        sparse_linear_set_plan(self.handle, rows_per_tile, splits)

    def set_union_plan(self, rows_per_tile: int = 0, workgroups: int = 0):
        sparse_linear_set_union_plan(self.handle, rows_per_tile, workgroups)

    def set_deterministic(self, on: bool = True):
        sparse_linear_set_deterministic(self.handle, on)

    def set_fused(self, on: bool = True):
        sparse_linear_set_fused(self.handle, on)

    def sync_status(self):
        """Synchronize the current stream; raise if a fused hand-off timed out."""
        sparse_linear_sync_status(self.handle, self._stream())

    def close(self):
        if getattr(self, "handle", None):
            sparse_linear_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# --------------------------------------------- Double Sparsity decode attention
def _stream_of(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def label_cache_update(key, label, channels, start=None, span=None) -> None:
    """Copy the label channels of key [B][H][S][d] (bf16) into label
    [B][H][S][r] for tokens start[b] .. start[b] + span - 1 (start: int32
    [B] on the device, or None for 0; span: default S)."""
    B, H, S, d = key.shape
    r = channels.shape[1]
    ds_label_cache_update(key.data_ptr(), label.data_ptr(), channels.data_ptr(),
                          0 if start is None else start.data_ptr(), B, H, S, d, r,
                          S if span is None else int(span), _stream_of(key))


def decode_attention(q, key, value, label, channels, seq_len, k: int, scale: Optional[float] = None,
                     out=None, tokens_out: bool = False):
    """One Double Sparsity decode step: q [B][H][d], key/value [B][H][S][d],
    label [B][H][S][r] (bf16), channels [H][r] and seq_len [B] (int32), all
    on one device. Returns out [B][H][d] fp32, or (out, tokens [B][H][k]
    int32) with tokens_out."""
    import torch
    B, H, S, d = key.shape
    r = channels.shape[1]
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    toks = torch.empty((B, H, k), dtype=torch.int32, device=q.device) if tokens_out else None
    ds_decode_attention(q.data_ptr(), key.data_ptr(), value.data_ptr(), 0 if label is None else label.data_ptr(),
                        channels.data_ptr(), seq_len.data_ptr(), B, H, S, d, r, k, float(scale), out.data_ptr(),
                        0 if toks is None else toks.data_ptr(), _stream_of(q))
    return (out, toks) if tokens_out else out
