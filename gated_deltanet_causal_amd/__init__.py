"""gated_deltanet_causal_amd -- the Gated DeltaNet sublayer hot path on MI355X.

A thin ctypes binding over ``libgdn.so`` (hand-written HIP for gfx950, C ABI in
``include/gdn.h``).  Every step of the path runs in the library's kernels;
this module only marshals torch device tensors (device memory and the current
stream) into the C calls and raises :class:`GDNError` on a failed status.
There is no CPU or PyTorch fallback: without the built library, importing the
binding's entry points raises.

Build the library with ``python -m gated_deltanet_causal_amd.build``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_SEQLENS, GDN_ERR_WORKSPACE, GDN_ERR_HIP = range(6)
GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2

# Every symbol include/gdn.h declares.
EXPORTS = ("gdn_abi_version", "gdn_status_string", "gdn_config_default", "gdn_conv1d_prefill",
           "gdn_conv1d_step", "gdn_chunk_prefill_workspace_size", "gdn_chunk_prefill",
           "gdn_chunk_prefill_ab", "gdn_gated_rmsnorm", "gdn_prefill_workspace_size", "gdn_prefill",
           "gdn_prefill_ab", "gdn_decode_step", "gdn_decode_step_ab", "gdn_verify_workspace_size",
           "gdn_verify", "gdn_verify_commit", "gdn_decode_step_h16", "gdn_state_convert",
           "gdn_chunk_prefill_noalloc")


class GDNError(RuntimeError):
    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call}: {message} (status {status})")
        self.status = status


class GDNConfig(ctypes.Structure):
    """Mirror of gdn_config_t."""
    _fields_ = [
        ("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
        ("conv_width", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("conv_act", ctypes.c_int32), ("decay_per_key_channel", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32),
        ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float), ("q_scale", ctypes.c_float),
    ]

    @property
    def conv_channels(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libgdn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libgdn.so not built at {path}; run python -m gated_deltanet_causal_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(GDNConfig)
    sig = {
        "gdn_abi_version": ([], ctypes.c_int),
        "gdn_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "gdn_config_default": ([cfgp], ctypes.c_int),
        "gdn_conv1d_prefill": ([cfgp, ctypes.c_int, vp, i64, vp, vp, vp, vp, i64, vp, vp, i32, i32, vp], ctypes.c_int),
        "gdn_conv1d_step": ([cfgp, ctypes.c_int, vp, i64, vp, vp, vp, i64, i32, vp], ctypes.c_int),
        "gdn_chunk_prefill_workspace_size": ([cfgp, i32, i32, ctypes.POINTER(sz)], ctypes.c_int),
        "gdn_chunk_prefill": ([cfgp, ctypes.c_int, ctypes.c_int, vp, vp, i64, vp, i64, vp, vp, vp, vp, vp,
                               i32, i32, vp, vp, vp, sz, vp], ctypes.c_int),
        "gdn_chunk_prefill_noalloc": ([cfgp, ctypes.c_int, ctypes.c_int, vp, vp, i64, vp, i64, vp, vp, vp, vp,
                                       vp, i32, i32, vp, vp, vp], ctypes.c_int),
        "gdn_gated_rmsnorm": ([cfgp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i64, vp], ctypes.c_int),
        "gdn_prefill_workspace_size": ([cfgp, ctypes.c_int, i32, i32, ctypes.POINTER(sz)], ctypes.c_int),
        "gdn_prefill": ([cfgp, ctypes.c_int, ctypes.c_int, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                         i32, i32, vp, vp, vp, sz, vp], ctypes.c_int),
        "gdn_decode_step": ([cfgp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp],
                            ctypes.c_int),
        "gdn_chunk_prefill_ab": ([cfgp, ctypes.c_int, ctypes.c_int, vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp,
                                  vp, i32, i32, vp, vp, vp, sz, vp], ctypes.c_int),
        "gdn_prefill_ab": ([cfgp, ctypes.c_int, ctypes.c_int, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                            vp, i32, i32, vp, vp, vp, sz, vp], ctypes.c_int),
        "gdn_decode_step_h16": ([cfgp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp],
                                ctypes.c_int),
        "gdn_state_convert": ([vp, ctypes.c_int, vp, ctypes.c_int, i64, vp], ctypes.c_int),
        "gdn_verify_workspace_size": ([cfgp, i32, i32, ctypes.POINTER(sz)], ctypes.c_int),
        "gdn_verify": ([cfgp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp],
                       ctypes.c_int),
        "gdn_verify_commit": ([cfgp, ctypes.c_int, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp], ctypes.c_int),
        "gdn_decode_step_ab": ([cfgp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(call: str, status: int) -> None:
    if status != GDN_OK:
        msg = load_library().gdn_status_string(status).decode()
        raise GDNError(call, status, msg)


def config(**overrides) -> GDNConfig:
    """gdn_config_default() with fields overridden by keyword."""
    cfg = GDNConfig()
    _check("gdn_config_default", load_library().gdn_config_default(ctypes.byref(cfg)))
    for k, v in overrides.items():
        if not hasattr(cfg, k):
            raise AttributeError(k)
        setattr(cfg, k, v)
    return cfg


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.float16:
        return GDN_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == GDN_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _row_stride(t: torch.Tensor) -> int:
    """Elements between rows of a [rows, ...] tensor whose inner dims are contiguous (an
    empty tensor, whose strides carry no layout, counts as packed rows)."""
    if t.numel() == 0:
        return math.prod(t.shape[1:]) if t.dim() > 1 else 0
    inner = 1
    for s, n in zip(reversed(t.stride()[1:]), reversed(t.shape[1:])):
        if s != inner:
            raise ValueError("inner dimensions must be contiguous")
        inner *= n
    return t.stride(0) if t.dim() > 1 else inner


def _cu_host(cu: torch.Tensor, cu_host) -> ctypes.Array:
    vals = cu.cpu().tolist() if cu_host is None else list(cu_host)
    return (ctypes.c_int32 * len(vals))(*vals)


_F32 = (torch.float32,)
_ACT = (torch.bfloat16, torch.float32)


def _need(t: Optional[torch.Tensor], name: str, dtypes, shape=None, contiguous: bool = True) -> None:
    """Raise ValueError unless t (when given) has one of dtypes, the given shape and is
    contiguous: the C ABI takes bare pointers and cannot check any of this itself."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_rows(t: torch.Tensor, name: str, dtypes, rows: int, width: int) -> None:
    """A [rows, ...] tensor (row stride free) whose rows hold `width` elements."""
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.dim() < 2 or t.shape[0] != rows or math.prod(t.shape[1:]) != width:
        raise ValueError(f"{name} must be [{rows}, {width}] (rows of {width} elements), got {tuple(t.shape)}")


def _need_gates(g, beta, lead, cfg: "GDNConfig", name: str = "") -> None:
    """g [*lead, Hv] (or [*lead, Hv, dk] with per-key-channel decay) and beta [*lead, Hv], fp32."""
    hv = cfg.num_v_heads
    gshape = (*lead, hv, cfg.head_k_dim) if cfg.decay_per_key_channel else (*lead, hv)
    _need(g, name + "g", _F32, gshape)
    _need(beta, name + "beta", _F32, (*lead, hv))


def _need_ab(ab, lead, act_dtype, cfg: "GDNConfig") -> None:
    if ab is None:
        return
    a, b, A_log, dt_bias = ab
    hv = cfg.num_v_heads
    _need(a, "a", (act_dtype,), (*lead, hv))
    _need(b, "b", (act_dtype,), (*lead, hv))
    _need(A_log, "A_log", _F32, (hv,))
    _need(dt_bias, "dt_bias", _F32, (hv,))


def _state_shape(n: int, cfg: "GDNConfig"):
    return (n, cfg.num_v_heads, cfg.head_v_dim, cfg.head_k_dim)


def conv1d_prefill(x: torch.Tensor, w: torch.Tensor, cu: torch.Tensor, *, cu_host=None,
                   conv_state_in: Optional[torch.Tensor] = None,
                   conv_state_out: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                   cfg: Optional[GDNConfig] = None) -> torch.Tensor:
    """x [T, Cc] (row stride free) -> y [T, Cc] in x's dtype; see gdn_conv1d_prefill."""
    cfg = cfg or config()
    T = x.shape[0]
    N = cu.numel() - 1
    Cc = cfg.conv_channels
    if y is None:
        y = torch.empty((T, Cc), dtype=x.dtype, device=x.device)
    _need_rows(x, "x", _ACT, T, Cc)
    _need_rows(y, "y", (x.dtype,), T, Cc)
    _need(w, "conv weight", _F32, (Cc, cfg.conv_width))
    _need(cu, "cu_seqlens", (torch.int32,), (N + 1,))
    _need(conv_state_in, "conv_state_in", (x.dtype,), (N, cfg.conv_width - 1, Cc))
    _need(conv_state_out, "conv_state_out", (x.dtype,), (N, cfg.conv_width - 1, Cc))
    hc = _cu_host(cu, cu_host)
    _check("gdn_conv1d_prefill", load_library().gdn_conv1d_prefill(
        ctypes.byref(cfg), _dtype(x), _ptr(x), _row_stride(x), _ptr(w), _ptr(conv_state_in),
        _ptr(conv_state_out), _ptr(y), _row_stride(y), _ptr(cu), hc, N, T, _stream()))
    return y


def conv1d_step(x: torch.Tensor, w: torch.Tensor, conv_state: torch.Tensor, *,
                y: Optional[torch.Tensor] = None, cfg: Optional[GDNConfig] = None) -> torch.Tensor:
    """x [B, Cc], conv_state [B, 3, Cc] (updated in place) -> y [B, Cc]."""
    cfg = cfg or config()
    B = x.shape[0]
    Cc = cfg.conv_channels
    if y is None:
        y = torch.empty((B, Cc), dtype=x.dtype, device=x.device)
    _need_rows(x, "x", _ACT, B, Cc)
    _need_rows(y, "y", (x.dtype,), B, Cc)
    _need(w, "conv weight", _F32, (Cc, cfg.conv_width))
    _need(conv_state, "conv_state", (x.dtype,), (B, cfg.conv_width - 1, Cc))
    _check("gdn_conv1d_step", load_library().gdn_conv1d_step(
        ctypes.byref(cfg), _dtype(x), _ptr(x), _row_stride(x), _ptr(w), _ptr(conv_state), _ptr(y),
        _row_stride(y), B, _stream()))
    return y


def chunk_prefill_workspace_size(N: int, T: int, cfg: Optional[GDNConfig] = None) -> int:
    cfg = cfg or config()
    out = ctypes.c_size_t(0)
    _check("gdn_chunk_prefill_workspace_size",
           load_library().gdn_chunk_prefill_workspace_size(ctypes.byref(cfg), N, T, ctypes.byref(out)))
    return out.value


def _gate_args(g, beta, ab):
    """(g, beta) given, or ab = (a, b, A_log, dt_bias) from which the kernels derive them."""
    if ab is None:
        return [_ptr(g), _ptr(beta)], False
    if g is not None or beta is not None:
        raise ValueError("pass either g and beta or ab=(a, b, A_log, dt_bias)")
    a, b, A_log, dt_bias = ab
    for t in (a, b, A_log, dt_bias):
        if not t.is_contiguous():
            raise ValueError("a, b, A_log and dt_bias must be contiguous")
    return [_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias)], True


def chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                  beta: Optional[torch.Tensor], cu: torch.Tensor, *, cu_host=None,
                  initial_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                  workspace: Optional[torch.Tensor] = None, cfg: Optional[GDNConfig] = None, ab=None):
    """Chunk-wise gated delta rule; q, k [T, Hk*dk] (or [T, Hk, dk]), v [T, Hv*dv], views with
    a shared row stride allowed.  Gates: g, beta, or (g = beta = None) ab = (a, b, A_log,
    dt_bias) with a, b [T, Hv] in q's dtype (gdn_chunk_prefill_ab).
    Returns (out [T, Hv, dv], final_state [N, Hv, dv, dk])."""
    cfg = cfg or config()
    T = q.shape[0]
    N = cu.numel() - 1
    hk, hv = cfg.num_k_heads, cfg.num_v_heads
    _need_rows(q, "q", _ACT, T, hk * cfg.head_k_dim)
    _need_rows(k, "k", (q.dtype,), T, hk * cfg.head_k_dim)
    _need_rows(v, "v", (q.dtype,), T, hv * cfg.head_v_dim)
    qs, ks = _row_stride(q), _row_stride(k)
    if qs != ks:
        raise ValueError("q and k must share a row stride")
    odt = out_dtype or q.dtype
    if out is None:
        out = torch.empty((T, cfg.num_v_heads, cfg.head_v_dim), dtype=odt, device=q.device)
    if final_state is None:
        final_state = torch.empty((N, cfg.num_v_heads, cfg.head_v_dim, cfg.head_k_dim),
                                  dtype=torch.float32, device=q.device)
    _need(cu, "cu_seqlens", (torch.int32,), (N + 1,))
    _need_gates(g, beta, (T,), cfg)
    _need_ab(ab, (T,), q.dtype, cfg)
    _need(initial_state, "initial_state", _F32, _state_shape(N, cfg))
    _need(final_state, "final_state", _F32, _state_shape(N, cfg))
    _need(out, "out", _ACT, (T, hv, cfg.head_v_dim))
    need = chunk_prefill_workspace_size(N, T, cfg)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", (torch.uint8,))
    hc = _cu_host(cu, cu_host)
    gates, derived = _gate_args(g, beta, ab)
    name = "gdn_chunk_prefill_ab" if derived else "gdn_chunk_prefill"
    _check(name, getattr(load_library(), name)(
        ctypes.byref(cfg), _dtype(q), _dtype(out), _ptr(q), _ptr(k), qs, _ptr(v), _row_stride(v),
        *gates, _ptr(initial_state), _ptr(cu), hc, N, T, _ptr(out), _ptr(final_state),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return out, final_state


def chunk_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, cu: torch.Tensor, *, cu_host=None,
                          initial_state: Optional[torch.Tensor] = None, out: torch.Tensor,
                          final_state: Optional[torch.Tensor] = None, cfg: Optional[GDNConfig] = None):
    """chunk_prefill with the library's fixed device scratch as the workspace
    (gdn_chunk_prefill_noalloc): the caller passes every output, nothing is allocated.
    Calls that overlap on one GPU race on the scratch."""
    cfg = cfg or config()
    T = q.shape[0]
    N = cu.numel() - 1
    hk, hv = cfg.num_k_heads, cfg.num_v_heads
    _need_rows(q, "q", _ACT, T, hk * cfg.head_k_dim)
    _need_rows(k, "k", (q.dtype,), T, hk * cfg.head_k_dim)
    _need_rows(v, "v", (q.dtype,), T, hv * cfg.head_v_dim)
    _need(cu, "cu_seqlens", (torch.int32,), (N + 1,))
    _need_gates(g, beta, (T,), cfg)
    _need(initial_state, "initial_state", _F32, _state_shape(N, cfg))
    _need(final_state, "final_state", _F32, _state_shape(N, cfg))
    _need(out, "out", _ACT, (T, hv, cfg.head_v_dim))
    qs, ks = _row_stride(q), _row_stride(k)
    if qs != ks:
        raise ValueError("q and k must share a row stride")
    hc = _cu_host(cu, cu_host)
    _check("gdn_chunk_prefill_noalloc", load_library().gdn_chunk_prefill_noalloc(
        ctypes.byref(cfg), _dtype(q), _dtype(out), _ptr(q), _ptr(k), qs, _ptr(v), _row_stride(v),
        _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu), hc, N, T, _ptr(out), _ptr(final_state),
        _stream()))
    return out, final_state


def gated_rmsnorm(o: torch.Tensor, z: torch.Tensor, w: torch.Tensor, *,
                  out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                  cfg: Optional[GDNConfig] = None) -> torch.Tensor:
    """o, z [rows, Hv, dv] -> sigmoid-gated RMSNorm output."""
    cfg = cfg or config()
    rows = o.shape[0]
    if out is None:
        out = torch.empty(o.shape, dtype=out_dtype or o.dtype, device=o.device)
    vshape = (rows, cfg.num_v_heads, cfg.head_v_dim)
    _need(o, "o", _ACT, vshape)
    _need(z, "z", _ACT, vshape)
    _need(out, "out", _ACT, vshape)
    _need(w, "norm weight", _F32, (cfg.head_v_dim,))
    _check("gdn_gated_rmsnorm", load_library().gdn_gated_rmsnorm(
        ctypes.byref(cfg), _dtype(o), _dtype(z), _dtype(out), _ptr(o), _ptr(z), _ptr(w), _ptr(out),
        rows, _stream()))
    return out


def prefill_workspace_size(N: int, T: int, dtype: torch.dtype = torch.bfloat16,
                           cfg: Optional[GDNConfig] = None) -> int:
    cfg = cfg or config()
    out = ctypes.c_size_t(0)
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    _check("gdn_prefill_workspace_size",
           load_library().gdn_prefill_workspace_size(ctypes.byref(cfg), code, N, T, ctypes.byref(out)))
    return out.value


def prefill(x: torch.Tensor, conv_w: torch.Tensor, cu: torch.Tensor, g: Optional[torch.Tensor],
            beta: Optional[torch.Tensor], z: torch.Tensor, norm_w: torch.Tensor, *, cu_host=None,
            conv_state_in: Optional[torch.Tensor] = None,
            conv_state_out: Optional[torch.Tensor] = None,
            initial_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            final_state: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
            workspace: Optional[torch.Tensor] = None, cfg: Optional[GDNConfig] = None, ab=None):
    """The whole sublayer prefill (conv -> chunk-wise delta rule -> gated norm) over packed
    sequences; x [T, Cc] (row stride free).  Gates: g, beta, or ab = (a, b, A_log, dt_bias)
    (gdn_prefill_ab).  Returns (out [T, Hv, dv], final_state)."""
    cfg = cfg or config()
    T = x.shape[0]
    N = cu.numel() - 1
    if out is None:
        out = torch.empty((T, cfg.num_v_heads, cfg.head_v_dim), dtype=out_dtype or x.dtype,
                          device=x.device)
    if final_state is None:
        final_state = torch.empty((N, cfg.num_v_heads, cfg.head_v_dim, cfg.head_k_dim),
                                  dtype=torch.float32, device=x.device)
    Cc, hv = cfg.conv_channels, cfg.num_v_heads
    _need_rows(x, "x", _ACT, T, Cc)
    _need(conv_w, "conv weight", _F32, (Cc, cfg.conv_width))
    _need(cu, "cu_seqlens", (torch.int32,), (N + 1,))
    _need(conv_state_in, "conv_state_in", (x.dtype,), (N, cfg.conv_width - 1, Cc))
    _need(conv_state_out, "conv_state_out", (x.dtype,), (N, cfg.conv_width - 1, Cc))
    _need_gates(g, beta, (T,), cfg)
    _need_ab(ab, (T,), x.dtype, cfg)
    _need(z, "z", (x.dtype,), (T, hv, cfg.head_v_dim))
    _need(norm_w, "norm weight", _F32, (cfg.head_v_dim,))
    _need(initial_state, "initial_state", _F32, _state_shape(N, cfg))
    _need(final_state, "final_state", _F32, _state_shape(N, cfg))
    _need(out, "out", _ACT, (T, hv, cfg.head_v_dim))
    _need(workspace, "workspace", (torch.uint8,))
    if workspace is None:
        workspace = torch.empty(prefill_workspace_size(N, T, x.dtype, cfg), dtype=torch.uint8,
                                device=x.device)
    hc = _cu_host(cu, cu_host)
    gates, derived = _gate_args(g, beta, ab)
    name = "gdn_prefill_ab" if derived else "gdn_prefill"
    _check(name, getattr(load_library(), name)(
        ctypes.byref(cfg), _dtype(x), _dtype(out), _ptr(x), _row_stride(x), _ptr(conv_w),
        _ptr(conv_state_in), _ptr(conv_state_out), *gates, _ptr(z), _ptr(norm_w),
        _ptr(initial_state), _ptr(cu), hc, N, T, _ptr(out), _ptr(final_state), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return out, final_state


def decode_step(x: torch.Tensor, conv_w: torch.Tensor, conv_state: torch.Tensor, g: Optional[torch.Tensor],
                beta: Optional[torch.Tensor], z: torch.Tensor, norm_w: torch.Tensor, state: torch.Tensor, *,
                out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                cfg: Optional[GDNConfig] = None, ab=None) -> torch.Tensor:
    """One fused decode step; conv_state and state are updated in place.  Gates: g, beta, or
    ab = (a, b, A_log, dt_bias) with a, b [B, Hv] in x's dtype (gdn_decode_step_ab).
    Returns out [B, Hv, dv]."""
    cfg = cfg or config()
    B = x.shape[0]
    if out is None:
        out = torch.empty((B, cfg.num_v_heads, cfg.head_v_dim), dtype=out_dtype or x.dtype, device=x.device)
    Cc, hv = cfg.conv_channels, cfg.num_v_heads
    _need(x, "x", _ACT, (B, Cc))
    _need(conv_w, "conv weight", _F32, (Cc, cfg.conv_width))
    _need(conv_state, "conv_state", (x.dtype,), (B, cfg.conv_width - 1, Cc))
    _need_gates(g, beta, (B,), cfg)
    _need_ab(ab, (B,), x.dtype, cfg)
    _need(z, "z", (x.dtype,), (B, hv, cfg.head_v_dim))
    _need(norm_w, "norm weight", _F32, (cfg.head_v_dim,))
    _need(state, "state", (torch.float32, torch.float16), _state_shape(B, cfg))
    _need(out, "out", _ACT, (B, hv, cfg.head_v_dim))
    gates, derived = _gate_args(g, beta, ab)
    if state.dtype == torch.float16:
        if derived:
            raise ValueError("the fp16-state decode takes g and beta")
        name = "gdn_decode_step_h16"
    else:
        name = "gdn_decode_step_ab" if derived else "gdn_decode_step"
    _check(name, getattr(load_library(), name)(
        ctypes.byref(cfg), _dtype(x), _dtype(out), _ptr(x), _ptr(conv_w), _ptr(conv_state), *gates,
        _ptr(z), _ptr(norm_w), _ptr(state), _ptr(out), B, _stream()))
    return out


def state_convert(src: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """A recurrent state widened (fp16 -> fp32) or narrowed (fp32 -> fp16, round to nearest even)."""
    _need(src, "state", (torch.float32, torch.float16))
    if dtype not in (torch.float32, torch.float16) or dtype == src.dtype:
        raise ValueError("state_convert converts between float32 and float16")
    dst = torch.empty(src.shape, dtype=dtype, device=src.device)
    _check("gdn_state_convert", load_library().gdn_state_convert(
        _ptr(src), _dtype(src), _ptr(dst), _dtype(dst), src.numel(), _stream()))
    return dst


def verify_workspace_size(B: int, K: int, cfg: Optional[GDNConfig] = None) -> int:
    cfg = cfg or config()
    out = ctypes.c_size_t(0)
    _check("gdn_verify_workspace_size",
           load_library().gdn_verify_workspace_size(ctypes.byref(cfg), B, K, ctypes.byref(out)))
    return out.value


def verify(x: torch.Tensor, conv_w: torch.Tensor, conv_state: torch.Tensor, g: torch.Tensor,
           beta: torch.Tensor, z: torch.Tensor, norm_w: torch.Tensor, state: torch.Tensor, *,
           out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
           workspace: Optional[torch.Tensor] = None, cfg: Optional[GDNConfig] = None):
    """Verify half of a speculative transaction: x [B, K, Cc], g / beta [B, K, Hv] (g
    [B, K, Hv, dk] per channel), z [B, K, Hv, dv].  conv_state and state are only read.
    Returns (out [B, K, Hv, dv], workspace); pass the workspace to verify_commit."""
    cfg = cfg or config()
    B, K = x.shape[0], x.shape[1]
    if out is None:
        out = torch.empty((B, K, cfg.num_v_heads, cfg.head_v_dim), dtype=out_dtype or x.dtype, device=x.device)
    Cc, hv = cfg.conv_channels, cfg.num_v_heads
    _need(x, "x", _ACT, (B, K, Cc))
    _need(conv_w, "conv weight", _F32, (Cc, cfg.conv_width))
    _need(conv_state, "conv_state", (x.dtype,), (B, cfg.conv_width - 1, Cc))
    _need_gates(g, beta, (B, K), cfg)
    _need(z, "z", (x.dtype,), (B, K, hv, cfg.head_v_dim))
    _need(norm_w, "norm weight", _F32, (cfg.head_v_dim,))
    _need(state, "state", _F32, _state_shape(B, cfg))
    _need(out, "out", _ACT, (B, K, hv, cfg.head_v_dim))
    _need(workspace, "workspace", (torch.uint8,))
    if workspace is None:
        workspace = torch.empty(verify_workspace_size(B, K, cfg), dtype=torch.uint8, device=x.device)
    _check("gdn_verify", load_library().gdn_verify(
        ctypes.byref(cfg), _dtype(x), _dtype(out), _ptr(x), _ptr(conv_w), _ptr(conv_state), _ptr(g), _ptr(beta),
        _ptr(z), _ptr(norm_w), _ptr(state), _ptr(out), B, K, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return out, workspace


def verify_commit(accepted: torch.Tensor, x: torch.Tensor, g: torch.Tensor, conv_state: torch.Tensor,
                  state: torch.Tensor, workspace: torch.Tensor, *, cfg: Optional[GDNConfig] = None) -> None:
    """Commit half: sequence b advances conv_state and state (in place) by its first
    clamp(accepted[b], 0, K) verified rows; accepted is an int32 device tensor [B]."""
    cfg = cfg or config()
    B, K = x.shape[0], x.shape[1]
    if accepted.dtype != torch.int32 or accepted.numel() != B:
        raise ValueError("accepted must be an int32 tensor of one entry per sequence")
    Cc = cfg.conv_channels
    _need(accepted, "accepted", (torch.int32,))
    _need(x, "x", _ACT, (B, K, Cc))
    _need_gates(g, None, (B, K), cfg)
    _need(conv_state, "conv_state", (x.dtype,), (B, cfg.conv_width - 1, Cc))
    _need(state, "state", _F32, _state_shape(B, cfg))
    _need(workspace, "workspace", (torch.uint8,))
    _check("gdn_verify_commit", load_library().gdn_verify_commit(
        ctypes.byref(cfg), _dtype(x), _ptr(accepted), _ptr(x), _ptr(g), _ptr(conv_state), _ptr(state), B, K,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))


def default_q_scale(cfg: GDNConfig) -> float:
    return cfg.q_scale if cfg.q_scale > 0 else 1.0 / math.sqrt(cfg.head_k_dim)
