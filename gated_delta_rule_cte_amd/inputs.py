"""Seeded synthetic inputs for the three GDN entry points.

This module only draws random numbers and casts them to the storage types the
entry points take (fp32, or bf16 rounded to nearest-even).  It holds none of
the recurrence's arithmetic, so both the HIP path and the CPU oracle can take
their inputs from here without sharing any of the method.

Every array is returned as an :class:`Arr`: the exact device representation
(``np.float32`` data, or ``np.uint16`` bit patterns for bf16) plus a helper to
widen it to float64 for the oracle.  Both sides therefore see identical bits.

Workload recipes follow the shapes and value distributions listed for the five
named workloads in :data:`WORKLOADS`; the seed for workload *i* is *i*
(``numpy.random.default_rng(i)``) and arrays are drawn in argument order.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Arr", "f32", "bf16", "cte_inputs", "tkg_inputs", "block_inputs",
           "WORKLOADS", "workload_inputs"]


# --------------------------------------------------------------------------
# storage casts (input preparation only)
# --------------------------------------------------------------------------
def _to_bf16_bits(x) -> np.ndarray:
    """float -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Goes through fp32 first; inputs are drawn in fp32/fp64 and never NaN.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Arr:
    """One input array in its device storage type."""

    data: np.ndarray  # float32, or uint16 bf16 bit patterns
    dtype: str        # "f32" or "bf16"

    @property
    def shape(self):
        return self.data.shape

    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return _bf16_bits_to_f32(self.data).astype(np.float64)
        return self.data.astype(np.float64)

    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return _bf16_bits_to_f32(self.data)
        return self.data.astype(np.float32, copy=False)


def f32(x) -> Arr:
    return Arr(np.ascontiguousarray(np.asarray(x, dtype=np.float32)), "f32")


def bf16(x) -> Arr:
    return Arr(_to_bf16_bits(x), "bf16")


def cast(x, dtype: str) -> Arr:
    return bf16(x) if dtype == "bf16" else f32(x)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    """Scale each last-axis vector to unit length (fp64), the stated
    precondition of the prefill's q and k."""
    x = x.astype(np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


# --------------------------------------------------------------------------
# per-entry-point generators
# --------------------------------------------------------------------------
def cte_inputs(B, Hk, Hv, S, Dk, Dv, dtype="bf16", g_range=(-0.3, -0.005),
               beta_range=(0.05, 0.95), state_std=None, seed=0):
    """Prefill inputs: q,k ~ N(0,1) made unit length per token, v ~ N(0,1),
    g_log ~ U(g_range), beta ~ U(beta_range), optional state ~ state_std*N(0,1).

    Returns a dict of :class:`Arr` plus the scalar ``scale = 1/sqrt(Dk)``.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hk, S, Dk), dtype=np.float32)
    k = rng.standard_normal((B, Hk, S, Dk), dtype=np.float32)
    v = rng.standard_normal((B, Hv, S, Dv), dtype=np.float32)
    g = rng.uniform(g_range[0], g_range[1], size=(B, Hv, S))
    beta = rng.uniform(beta_range[0], beta_range[1], size=(B, Hv, S))
    out = dict(query=cast(_unit_rows(q), dtype), key=cast(_unit_rows(k), dtype),
               value=cast(v, dtype), g_log=f32(g), beta=f32(beta),
               scale=float(1.0 / np.sqrt(Dk)))
    if state_std is not None:
        out["recurrent_state"] = f32(state_std * rng.standard_normal((B, Hv, Dk, Dv)))
    return out


def cte_fused_inputs(B, Hk, Hv, S, Dk, Dv, dtype="bf16", A_range=(0.02, 0.2), state_std=None, seed=0):
    """Inputs of the prefill with the decode step's gates and norm: raw q, k, v,
    z ~ N(0,1); b, a ~ N(0,1) fp32 per token of every value head;
    A_log = log U(A_range), dt_bias ~ U(-1,1) per value head (A_range keeps the
    per-token decay g = -exp(A_log) softplus(a + dt_bias) near the prefill
    workloads' U(-0.3, -0.005)); norm_weight = 1 + 0.1 N(0,1); optional state
    ~ state_std*N(0,1)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hk, S, Dk), dtype=np.float32)
    k = rng.standard_normal((B, Hk, S, Dk), dtype=np.float32)
    v = rng.standard_normal((B, Hv, S, Dv), dtype=np.float32)
    z = rng.standard_normal((B, Hv, S, Dv), dtype=np.float32)
    b = rng.standard_normal((B, Hv, S))
    a = rng.standard_normal((B, Hv, S))
    A_log = np.log(rng.uniform(A_range[0], A_range[1], size=Hv))
    dt_bias = rng.uniform(-1.0, 1.0, size=Hv)
    norm_weight = 1.0 + 0.1 * rng.standard_normal(Dv)
    out = dict(q=cast(q, dtype), k=cast(k, dtype), v=cast(v, dtype), z=cast(z, dtype),
               b=f32(b), a=f32(a), A_log=f32(A_log), dt_bias=f32(dt_bias), norm_weight=f32(norm_weight))
    if state_std is not None:
        out["recurrent_state"] = f32(state_std * rng.standard_normal((B, Hv, Dk, Dv)))
    return out


def _head_params(rng, Hv, V):
    A_log = np.log(rng.uniform(1.0, 16.0, size=Hv))
    dt_bias = rng.uniform(-1.0, 1.0, size=Hv)
    norm_weight = 1.0 + 0.1 * rng.standard_normal(V)
    return f32(A_log), f32(dt_bias), f32(norm_weight)


def tkg_inputs(B, Hv, K, V, dtype="bf16", state_std=0.05, seed=1):
    """Decode-step inputs with BH = B*Hv (heads cycling fastest per batch):
    raw q,k,v,z ~ N(0,1); b,a ~ N(0,1) fp32; A_log = log U(1,16);
    dt_bias ~ U(-1,1); norm_weight = 1 + 0.1 N(0,1); state ~ state_std*N(0,1)."""
    rng = np.random.default_rng(seed)
    BH = B * Hv
    q = rng.standard_normal((BH, K), dtype=np.float32)
    k = rng.standard_normal((BH, K), dtype=np.float32)
    v = rng.standard_normal((BH, V), dtype=np.float32)
    z = rng.standard_normal((BH, V), dtype=np.float32)
    b = rng.standard_normal(BH)
    a = rng.standard_normal(BH)
    A_log, dt_bias, norm_weight = _head_params(rng, Hv, V)
    state = state_std * rng.standard_normal((BH, K, V), dtype=np.float32)
    return dict(q=cast(q, dtype), k=cast(k, dtype), v=cast(v, dtype), z=cast(z, dtype),
                b=f32(b), a=f32(a), A_log=A_log, dt_bias=dt_bias,
                norm_weight=norm_weight, state_in=f32(state), num_v_heads=Hv)


def block_inputs(B, H, Hk, Hv, Dk, Dv, K_win=4, w_std=0.02, conv_w_std=0.5,
                 state_std=0.05, seed=4):
    """Fused decode-layer inputs: hidden ~ N(0,1) bf16; in_proj weights ~
    N(0, w_std) bf16 stored [H, N]; conv weight ~ N(0, conv_w_std) fp32;
    conv window ~ N(0,1) bf16; per-head parameters as for the decode step;
    recurrent state ~ state_std*N(0,1) fp32."""
    rng = np.random.default_rng(seed)
    key_dim, value_dim = Hk * Dk, Hv * Dv
    conv_dim = 2 * key_dim + value_dim
    hidden = rng.standard_normal((B, 1, H), dtype=np.float32)
    W_qkv = w_std * rng.standard_normal((H, conv_dim), dtype=np.float32)
    W_z = w_std * rng.standard_normal((H, value_dim), dtype=np.float32)
    W_a = w_std * rng.standard_normal((H, Hv), dtype=np.float32)
    W_b = w_std * rng.standard_normal((H, Hv), dtype=np.float32)
    conv_w = conv_w_std * rng.standard_normal((conv_dim, K_win), dtype=np.float32)
    conv_state = rng.standard_normal((B, conv_dim, K_win), dtype=np.float32)
    A_log, dt_bias, norm_weight = _head_params(rng, Hv, Dv)
    state = state_std * rng.standard_normal((B, Hv, Dk, Dv), dtype=np.float32)
    return dict(hidden=bf16(hidden), W_in_qkv=bf16(W_qkv), W_in_z=bf16(W_z),
                W_in_a=bf16(W_a), W_in_b=bf16(W_b), conv_weight=f32(conv_w),
                conv_state=bf16(conv_state), A_log=A_log, dt_bias=dt_bias,
                norm_weight=norm_weight, recurrent_state=f32(state),
                num_k_heads=Hk, num_v_heads=Hv, head_k_dim=Dk, head_v_dim=Dv)


def block_cte_inputs(B, S, H, Hk, Hv, Dk, Dv, K_win=4, w_std=0.02, conv_w_std=0.5,
                     A_range=(0.02, 0.2), state_std=0.05, seed=5):
    """Prefill-layer inputs: hidden [B, S, H] ~ N(0,1) bf16 and the decode
    layer's weights and windows; A_log = log U(A_range) per value head keeps the
    per-token decay near the prefill workloads' range (as in cte_fused_inputs);
    dt_bias ~ U(-1,1); norm_weight = 1 + 0.1 N(0,1)."""
    rng = np.random.default_rng(seed)
    key_dim, value_dim = Hk * Dk, Hv * Dv
    conv_dim = 2 * key_dim + value_dim
    hidden = rng.standard_normal((B, S, H), dtype=np.float32)
    W_qkv = w_std * rng.standard_normal((H, conv_dim), dtype=np.float32)
    W_z = w_std * rng.standard_normal((H, value_dim), dtype=np.float32)
    W_a = w_std * rng.standard_normal((H, Hv), dtype=np.float32)
    W_b = w_std * rng.standard_normal((H, Hv), dtype=np.float32)
    conv_w = conv_w_std * rng.standard_normal((conv_dim, K_win), dtype=np.float32)
    conv_state = rng.standard_normal((B, conv_dim, K_win), dtype=np.float32)
    A_log = np.log(rng.uniform(A_range[0], A_range[1], size=Hv))
    dt_bias = rng.uniform(-1.0, 1.0, size=Hv)
    norm_weight = 1.0 + 0.1 * rng.standard_normal(Dv)
    state = state_std * rng.standard_normal((B, Hv, Dk, Dv), dtype=np.float32)
    return dict(hidden=bf16(hidden), W_in_qkv=bf16(W_qkv), W_in_z=bf16(W_z),
                W_in_a=bf16(W_a), W_in_b=bf16(W_b), conv_weight=f32(conv_w),
                conv_state=bf16(conv_state), A_log=f32(A_log), dt_bias=f32(dt_bias),
                norm_weight=f32(norm_weight), recurrent_state=f32(state),
                num_k_heads=Hk, num_v_heads=Hv, head_k_dim=Dk, head_v_dim=Dv)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
WORKLOADS = {
    # small fp32 prefill the oracle finishes instantly
    "cte_fp32_b1_h2_s128_d64": dict(
        kind="cte", seed=0, B=1, Hk=2, Hv=2, S=128, Dk=64, Dv=64, dtype="f32",
        g_range=(-0.5, -0.01), state_std=None),
    # decode step, BH = 32*32 = 1024, K = V = 128
    "tkg_b32_hv32_d128": dict(kind="tkg", seed=1, B=32, Hv=32, K=128, V=128),
    # GQA prefill, S = 4096, supplied state updated in place
    "cte_bf16_b1_hk16_hv32_s4096_d128": dict(
        kind="cte", seed=2, B=1, Hk=16, Hv=32, S=4096, Dk=128, Dv=128, dtype="bf16",
        g_range=(-0.3, -0.005), state_std=0.05),
    # long batched prefill, zero initial state
    "cte_bf16_b4_hk16_hv32_s16384_d128": dict(
        kind="cte", seed=3, B=4, Hk=16, Hv=32, S=16384, Dk=128, Dv=128, dtype="bf16",
        g_range=(-0.3, -0.005), state_std=None),
    # fused decode layer, B = 64, H = 2048
    "block_b64_h2048_hk16_hv32_d128": dict(
        kind="block", seed=4, B=64, H=2048, Hk=16, Hv=32, Dk=128, Dv=128, K_win=4),
}


def workload_inputs(name: str, **override):
    w = dict(WORKLOADS[name])
    w.update(override)
    kind = w.pop("kind")
    if kind == "cte":
        return cte_inputs(w["B"], w["Hk"], w["Hv"], w["S"], w["Dk"], w["Dv"],
                          dtype=w["dtype"], g_range=w["g_range"],
                          state_std=w["state_std"], seed=w["seed"])
    if kind == "tkg":
        return tkg_inputs(w["B"], w["Hv"], w["K"], w["V"], seed=w["seed"])
    return block_inputs(w["B"], w["H"], w["Hk"], w["Hv"], w["Dk"], w["Dv"],
                        K_win=w["K_win"], seed=w["seed"])
