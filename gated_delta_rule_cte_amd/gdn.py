"""Thin Python binding over libgdn (include/gdn.h).

Argument marshalling only: shapes are read from torch tensors, outputs are
allocated with torch, and every computation runs in the HIP kernels of
``libgdn.so``.  The library must be built (``python -m
gated_delta_rule_cte_amd.build``); there is no fallback of any kind, and a
missing library or a non-zero status raises.

Function names and argument order follow the pages ("GDN CTE Kernel API
Reference" gdn_cte, "GDN TKG Kernel API Reference" gdn_tkg, "GDN Block TKG
Kernel API Reference" gdn_block_tkg).
"""
from __future__ import annotations

import ctypes
import os

# GDN_LIBRARY selects another build of the same library (for instance the
# host-sanitized one that tests/sanitize_host.py builds)
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
GDN_CTE_ALGO_DEFAULT = 0
GDN_CTE_ALGO_NEUMANN = 1
STATUS = {0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_DTYPE",
          -4: "GDN_ERR_ALIGN", -5: "GDN_ERR_ALIAS", -6: "GDN_ERR_WORKSPACE",
          -7: "GDN_ERR_UNSUPPORTED", -8: "GDN_ERR_LAUNCH", -9: "GDN_ERR_DEVICE"}

#: every symbol include/gdn.h declares
EXPORTS = ("gdn_cte", "gdn_cte_workspace_size", "gdn_cte_noalloc", "gdn_cte_fused", "gdn_cte_fused_workspace_size",
           "gdn_block_cte", "gdn_block_cte_workspace_size", "gdn_tkg", "gdn_block_tkg",
           "gdn_block_tkg_workspace_size", "gdn_status_string", "gdn_last_error",
           "gdn_version")

_lib = None


class GdnError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libgdn.so and declare its C signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m gated_delta_rule_cte_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gdn_cte.argtypes = [P, P, P, P, P, F, P, I, P, I, I, I, I, I, I, I, I, P, Z, P]
    lib.gdn_cte.restype = I
    lib.gdn_cte_workspace_size.argtypes = [I] * 7
    lib.gdn_cte_workspace_size.restype = Z
    lib.gdn_cte_noalloc.argtypes = [P, P, P, P, P, F, P, I, P, I, I, I, I, I, I, I, I, P]
    lib.gdn_cte_noalloc.restype = I
    lib.gdn_cte_fused.argtypes = [P] * 10 + [I, P] + [I] * 8 + [F, P, Z, P]
    lib.gdn_cte_fused.restype = I
    lib.gdn_cte_fused_workspace_size.argtypes = [I] * 7
    lib.gdn_cte_fused_workspace_size.restype = Z
    lib.gdn_block_cte.argtypes = [P] * 14 + [I] * 9 + [F, P, Z, P]
    lib.gdn_block_cte.restype = I
    lib.gdn_block_cte_workspace_size.argtypes = [I] * 8
    lib.gdn_block_cte_workspace_size.restype = Z
    lib.gdn_tkg.argtypes = [P] * 12 + [I, I, I, I, I, F, P]
    lib.gdn_tkg.restype = I
    lib.gdn_block_tkg.argtypes = [P] * 14 + [I] * 7 + [F, P, Z, P]
    lib.gdn_block_tkg.restype = I
    lib.gdn_block_tkg_workspace_size.argtypes = [I] * 7
    lib.gdn_block_tkg_workspace_size.restype = Z
    lib.gdn_status_string.argtypes = [I]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_version.argtypes = []
    lib.gdn_version.restype = I
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise GdnError(status, _lib.gdn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _req(t, name, dtype=None, shape=None):
    """Type, dtype, shape and contiguity of one argument (the device is checked
    separately by _on_gpu, after every argument's shape)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_gpu(named):
    """Every tensor on the same GPU device; returns that device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")
    return dev


def _workspace(t, name="workspace"):
    import torch
    _req(t, name, torch.uint8)
    if t.dim() != 1:
        raise ValueError(f"{name} must be one-dimensional (bytes)")
    return t


def gdn_cte(query, key, value, g_log, beta, scale=1.0, recurrent_state=None,
            algorithm=GDN_CTE_ALGO_DEFAULT, out=None):
    """Chunked GDN prefill.  Returns (out [B,Hv,S,Dv], state [B,Hv,Dk,Dv] fp32).

    With ``recurrent_state`` given it is the initial state and is updated in
    place (and returned); otherwise a new zero-initialised-by-definition state
    buffer is allocated and never read by the kernel."""
    import torch
    lib = load()
    B, Hk, S, Dk = query.shape
    Hv, Dv = value.shape[1], value.shape[3]
    _req(query, "query")
    _req(key, "key", query.dtype, (B, Hk, S, Dk))
    _req(value, "value", query.dtype, (B, Hv, S, Dv))
    _req(g_log, "g_log", torch.float32, (B, Hv, S))
    _req(beta, "beta", torch.float32, (B, Hv, S))
    has_init = recurrent_state is not None
    if has_init:
        _req(recurrent_state, "recurrent_state", torch.float32, (B, Hv, Dk, Dv))
    if out is not None:
        _req(out, "out", query.dtype, (B, Hv, S, Dv))
    dev = _on_gpu([("query", query), ("key", key), ("value", value), ("g_log", g_log), ("beta", beta),
                   ("recurrent_state", recurrent_state), ("out", out)])
    state = recurrent_state if has_init else torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((B, Hv, S, Dv), dtype=query.dtype, device=dev)
    dt = _dtype_code(query)
    ws_bytes = lib.gdn_cte_workspace_size(B, Hk, Hv, S, Dk, Dv, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    _check(lib.gdn_cte(_ptr(query), _ptr(key), _ptr(value), _ptr(g_log), _ptr(beta),
                       float(scale), _ptr(state), int(has_init), _ptr(out),
                       B, Hk, Hv, S, Dk, Dv, dt, int(algorithm), _ptr(ws), ws_bytes,
                       _stream(dev)))
    return out, state


def gdn_cte_noalloc(query, key, value, g_log, beta, scale, recurrent_state, out,
                    has_initial_state=True, algorithm=GDN_CTE_ALGO_DEFAULT):
    """gdn_cte on the library's fixed scratch (no device allocation anywhere:
    the caller passes every output).  ``recurrent_state`` [B,Hv,Dk,Dv] fp32 is
    read as the initial state when ``has_initial_state`` and receives the
    final state; ``out`` [B,Hv,S,Dv].  Returns (out, recurrent_state)."""
    import torch
    lib = load()
    B, Hk, S, Dk = query.shape
    Hv, Dv = value.shape[1], value.shape[3]
    _req(query, "query")
    _req(key, "key", query.dtype, (B, Hk, S, Dk))
    _req(value, "value", query.dtype, (B, Hv, S, Dv))
    _req(g_log, "g_log", torch.float32, (B, Hv, S))
    _req(beta, "beta", torch.float32, (B, Hv, S))
    _req(recurrent_state, "recurrent_state", torch.float32, (B, Hv, Dk, Dv))
    _req(out, "out", query.dtype, (B, Hv, S, Dv))
    dev = _on_gpu([("query", query), ("key", key), ("value", value), ("g_log", g_log), ("beta", beta),
                   ("recurrent_state", recurrent_state), ("out", out)])
    _check(lib.gdn_cte_noalloc(_ptr(query), _ptr(key), _ptr(value), _ptr(g_log), _ptr(beta), float(scale),
                               _ptr(recurrent_state), int(bool(has_initial_state)), _ptr(out),
                               B, Hk, Hv, S, Dk, Dv, _dtype_code(query), int(algorithm), _stream(dev)))
    return out, recurrent_state


def gdn_cte_fused(q, k, v, b, a, A_log, dt_bias, z, norm_weight, recurrent_state=None,
                  algorithm=GDN_CTE_ALGO_DEFAULT, rms_eps=1e-6, out=None):
    """Chunked prefill with the decode step's gates and output norm: RAW q, k
    [B,Hk,S,Dk]; v, z [B,Hv,S,Dv]; b, a [B,Hv,S] fp32; A_log, dt_bias [Hv];
    norm_weight [Dv].  Returns (out [B,Hv,S,Dv] = RMSNormGated(o, z), state
    [B,Hv,Dk,Dv] fp32); a given ``recurrent_state`` is the initial state and is
    updated in place."""
    import torch
    lib = load()
    B, Hk, S, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[3]
    _req(q, "q")
    _req(k, "k", q.dtype, (B, Hk, S, Dk))
    _req(v, "v", q.dtype, (B, Hv, S, Dv))
    _req(z, "z", q.dtype, (B, Hv, S, Dv))
    _req(b, "b", torch.float32, (B, Hv, S))
    _req(a, "a", torch.float32, (B, Hv, S))
    _req(A_log, "A_log", torch.float32, (Hv,))
    _req(dt_bias, "dt_bias", torch.float32, (Hv,))
    _req(norm_weight, "norm_weight", torch.float32, (Dv,))
    has_init = recurrent_state is not None
    if has_init:
        _req(recurrent_state, "recurrent_state", torch.float32, (B, Hv, Dk, Dv))
    if out is not None:
        _req(out, "out", q.dtype, (B, Hv, S, Dv))
    dev = _on_gpu([("q", q), ("k", k), ("v", v), ("z", z), ("b", b), ("a", a), ("A_log", A_log),
                   ("dt_bias", dt_bias), ("norm_weight", norm_weight), ("recurrent_state", recurrent_state),
                   ("out", out)])
    state = recurrent_state if has_init else torch.empty((B, Hv, Dk, Dv), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((B, Hv, S, Dv), dtype=q.dtype, device=dev)
    dt = _dtype_code(q)
    ws_bytes = lib.gdn_cte_fused_workspace_size(B, Hk, Hv, S, Dk, Dv, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    _check(lib.gdn_cte_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(b), _ptr(a), _ptr(A_log), _ptr(dt_bias),
                             _ptr(z), _ptr(norm_weight), _ptr(state), int(has_init), _ptr(out),
                             B, Hk, Hv, S, Dk, Dv, dt, int(algorithm), float(rms_eps), _ptr(ws), ws_bytes,
                             _stream(dev)))
    return out, state


def gdn_block_cte(hidden, W_in_qkv, W_in_z, W_in_a, W_in_b, conv_weight, conv_state,
                  A_log, dt_bias, norm_weight, recurrent_state, algorithm=GDN_CTE_ALGO_DEFAULT,
                  rms_eps=1e-6, conv_state_out=None, recurrent_state_out=None, out=None):
    """Prefill layer over S tokens: hidden [B,S,H] bf16 -> (out [B,S,value_dim]
    bf16, conv_state' [B,conv_dim,K_win] bf16, recurrent_state' [B,Hv,Dk,Dv]
    fp32).  Functional by default; pass ``conv_state_out=conv_state`` and/or
    ``recurrent_state_out=recurrent_state`` to update the caches in place.  All
    dimensions come from the tensor shapes, as for gdn_block_tkg."""
    import torch
    lib = load()
    B, S, H = hidden.shape
    conv_dim = W_in_qkv.shape[1]
    value_dim = W_in_z.shape[1]
    Hv = W_in_a.shape[1]
    K_win = conv_weight.shape[1]
    _, _, Dk, Dv = recurrent_state.shape
    key_dim = (conv_dim - value_dim) // 2
    Hk = key_dim // Dk
    bf = torch.bfloat16
    _req(hidden, "hidden", bf)
    _req(W_in_qkv, "W_in_qkv", bf, (H, conv_dim))
    _req(W_in_z, "W_in_z", bf, (H, value_dim))
    _req(W_in_a, "W_in_a", bf, (H, Hv))
    _req(W_in_b, "W_in_b", bf, (H, Hv))
    _req(conv_weight, "conv_weight", torch.float32, (conv_dim, K_win))
    _req(conv_state, "conv_state", bf, (B, conv_dim, K_win))
    _req(A_log, "A_log", torch.float32, (Hv,))
    _req(dt_bias, "dt_bias", torch.float32, (Hv,))
    _req(norm_weight, "norm_weight", torch.float32, (Dv,))
    _req(recurrent_state, "recurrent_state", torch.float32, (B, Hv, Dk, Dv))
    if value_dim != Hv * Dv or key_dim * 2 + value_dim != conv_dim or Hk * Dk != key_dim:
        raise ValueError("inconsistent block shapes")
    if out is not None:
        _req(out, "out", bf, (B, S, value_dim))
    if conv_state_out is not None:
        _req(conv_state_out, "conv_state_out", bf, (B, conv_dim, K_win))
    if recurrent_state_out is not None:
        _req(recurrent_state_out, "recurrent_state_out", torch.float32, (B, Hv, Dk, Dv))
    dev = _on_gpu([("hidden", hidden), ("W_in_qkv", W_in_qkv), ("W_in_z", W_in_z), ("W_in_a", W_in_a),
                   ("W_in_b", W_in_b), ("conv_weight", conv_weight), ("conv_state", conv_state), ("A_log", A_log),
                   ("dt_bias", dt_bias), ("norm_weight", norm_weight), ("recurrent_state", recurrent_state),
                   ("out", out), ("conv_state_out", conv_state_out), ("recurrent_state_out", recurrent_state_out)])
    if out is None:
        out = torch.empty((B, S, value_dim), dtype=bf, device=dev)
    if conv_state_out is None:
        conv_state_out = torch.empty_like(conv_state)
    if recurrent_state_out is None:
        recurrent_state_out = torch.empty_like(recurrent_state)
    ws_bytes = lib.gdn_block_cte_workspace_size(B, S, H, Hk, Hv, Dk, Dv, K_win)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    _check(lib.gdn_block_cte(_ptr(hidden), _ptr(W_in_qkv), _ptr(W_in_z), _ptr(W_in_a), _ptr(W_in_b),
                             _ptr(conv_weight), _ptr(conv_state), _ptr(A_log), _ptr(dt_bias),
                             _ptr(norm_weight), _ptr(recurrent_state), _ptr(out), _ptr(conv_state_out),
                             _ptr(recurrent_state_out), B, S, H, Hk, Hv, Dk, Dv, K_win, int(algorithm),
                             float(rms_eps), _ptr(ws), ws_bytes, _stream(dev)))
    return out, conv_state_out, recurrent_state_out


def gdn_tkg(q, k, v, b, a, A_log, dt_bias, z, norm_weight, state_in,
            state_out=None, rms_eps=1e-6, out=None):
    """Fused single-token GDN decode step.  Returns (out [BH,V] bf16,
    state_out [BH,K,V] fp32).  Pass ``state_out=state_in`` to update in place."""
    import torch
    lib = load()
    BH, K = q.shape
    V = v.shape[1]
    Hv = A_log.shape[0]
    _req(q, "q")
    for name, t, shp in (("k", k, (BH, K)), ("v", v, (BH, V)), ("z", z, (BH, V))):
        _req(t, name, q.dtype, shp)
    for name, t, shp in (("b", b, (BH,)), ("a", a, (BH,)), ("A_log", A_log, (Hv,)),
                         ("dt_bias", dt_bias, (Hv,)), ("norm_weight", norm_weight, (V,)),
                         ("state_in", state_in, (BH, K, V))):
        _req(t, name, torch.float32, shp)
    if state_out is not None:
        _req(state_out, "state_out", torch.float32, (BH, K, V))
    if out is not None:
        _req(out, "out", torch.bfloat16, (BH, V))
    dev = _on_gpu([("q", q), ("k", k), ("v", v), ("z", z), ("b", b), ("a", a), ("A_log", A_log),
                   ("dt_bias", dt_bias), ("norm_weight", norm_weight), ("state_in", state_in),
                   ("state_out", state_out), ("out", out)])
    if state_out is None:
        state_out = torch.empty_like(state_in)
    if out is None:
        out = torch.empty((BH, V), dtype=torch.bfloat16, device=dev)
    _check(lib.gdn_tkg(_ptr(q), _ptr(k), _ptr(v), _ptr(b), _ptr(a), _ptr(A_log), _ptr(dt_bias),
                       _ptr(z), _ptr(norm_weight), _ptr(state_in), _ptr(state_out), _ptr(out),
                       BH, Hv, K, V, _dtype_code(q), float(rms_eps), _stream(dev)))
    return out, state_out


def block_workspace_bytes(B, H, num_k_heads, num_v_heads, head_k_dim, head_v_dim, K_win):
    return load().gdn_block_tkg_workspace_size(B, H, num_k_heads, num_v_heads, head_k_dim,
                                               head_v_dim, K_win)


def gdn_block_tkg(hidden, W_in_qkv, W_in_z, W_in_a, W_in_b, conv_weight, conv_state,
                  A_log, dt_bias, norm_weight, recurrent_state, rms_eps=1e-6,
                  conv_state_out=None, recurrent_state_out=None, out=None, workspace=None):
    """Fused GDN decode layer.  Returns (out [B,1,value_dim] bf16,
    conv_state' [B,conv_dim,K_win] bf16, recurrent_state' [B,Hv,Dk,Dv] fp32).

    Functional by default (new output buffers); pass ``conv_state_out=conv_state``
    and/or ``recurrent_state_out=recurrent_state`` to update the caches in place.
    All dimensions come from the tensor shapes."""
    import torch
    lib = load()
    B, _, H = hidden.shape
    conv_dim = W_in_qkv.shape[1]
    value_dim = W_in_z.shape[1]
    Hv = W_in_a.shape[1]
    K_win = conv_weight.shape[1]
    _, _, Dk, Dv = recurrent_state.shape
    key_dim = (conv_dim - value_dim) // 2
    Hk = key_dim // Dk
    bf = torch.bfloat16
    _req(hidden, "hidden", bf)
    _req(W_in_qkv, "W_in_qkv", bf, (H, conv_dim))
    _req(W_in_z, "W_in_z", bf, (H, value_dim))
    _req(W_in_a, "W_in_a", bf, (H, Hv))
    _req(W_in_b, "W_in_b", bf, (H, Hv))
    _req(conv_weight, "conv_weight", torch.float32, (conv_dim, K_win))
    _req(conv_state, "conv_state", bf, (B, conv_dim, K_win))
    _req(A_log, "A_log", torch.float32, (Hv,))
    _req(dt_bias, "dt_bias", torch.float32, (Hv,))
    _req(norm_weight, "norm_weight", torch.float32, (Dv,))
    _req(recurrent_state, "recurrent_state", torch.float32, (B, Hv, Dk, Dv))
    if value_dim != Hv * Dv or key_dim * 2 + value_dim != conv_dim or Hk * Dk != key_dim:
        raise ValueError("inconsistent block shapes")
    if out is not None:
        _req(out, "out", bf, (B, 1, value_dim))
    if conv_state_out is not None:
        _req(conv_state_out, "conv_state_out", bf, (B, conv_dim, K_win))
    if recurrent_state_out is not None:
        _req(recurrent_state_out, "recurrent_state_out", torch.float32, (B, Hv, Dk, Dv))
    if workspace is not None:
        _workspace(workspace)
    dev = _on_gpu([("hidden", hidden), ("W_in_qkv", W_in_qkv), ("W_in_z", W_in_z), ("W_in_a", W_in_a),
                   ("W_in_b", W_in_b), ("conv_weight", conv_weight), ("conv_state", conv_state), ("A_log", A_log),
                   ("dt_bias", dt_bias), ("norm_weight", norm_weight), ("recurrent_state", recurrent_state),
                   ("out", out), ("conv_state_out", conv_state_out), ("recurrent_state_out", recurrent_state_out),
                   ("workspace", workspace)])
    if conv_state_out is None:
        conv_state_out = torch.empty_like(conv_state)
    if recurrent_state_out is None:
        recurrent_state_out = torch.empty_like(recurrent_state)
    if out is None:
        out = torch.empty((B, 1, value_dim), dtype=bf, device=dev)
    ws_bytes = lib.gdn_block_tkg_workspace_size(B, H, Hk, Hv, Dk, Dv, K_win)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(lib.gdn_block_tkg(_ptr(hidden), _ptr(W_in_qkv), _ptr(W_in_z), _ptr(W_in_a),
                             _ptr(W_in_b), _ptr(conv_weight), _ptr(conv_state), _ptr(A_log),
                             _ptr(dt_bias), _ptr(norm_weight), _ptr(recurrent_state), _ptr(out),
                             _ptr(conv_state_out), _ptr(recurrent_state_out), B, H, Hk, Hv, Dk, Dv,
                             K_win, float(rms_eps), _ptr(workspace), workspace.numel(),
                             _stream(dev)))
    return out, conv_state_out, recurrent_state_out


# short aliases
cte = gdn_cte
tkg = gdn_tkg
block_tkg = gdn_block_tkg
