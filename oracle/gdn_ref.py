"""CPU oracle for the gated delta-rule (GDN) prefill and decode paths.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may call it.  It shares no code with the HIP library.

Everything is evaluated token by token in float64, the plain definition of the
recurrence with no chunking, blocking or reordering.  The inputs are the exact
values the device receives (bf16 inputs already widened), so the only
difference from the device is arithmetic precision and evaluation order.

The recurrence (the gated delta rule of Yang, Kautz & Hatamizadeh, "Gated Delta
Networks: Improving Mamba2 with Delta Rule", ICLR 2025), per value head, with an
fp32 state S of shape [Dk, Dv]:

    S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t

The pages ("GDN CTE Kernel API Reference", "GDN TKG Kernel API Reference",
"GDN Block TKG Kernel API Reference") fix the interfaces, layouts, the GQA head
map and the operators around the core.  Readings taken where they are silent
are listed next to each function.

Pinned by tests/test_oracle_pins.py (brute force, closed forms, invariants and
library routines), not by retyping these formulas.
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_round", "l2norm", "sigmoid", "softplus", "silu",
           "rms_norm_gated", "cte", "cte_fused", "tkg", "conv1d_decode", "in_proj",
           "block_tkg", "conv1d_prefill", "block_cte", "L2_EPS", "RMS_EPS"]

#: epsilon inside the l2 norm: x / sqrt(sum(x^2) + L2_EPS).  The TKG page names
#: "l2norm(q,k)" without a formula; this is the plain reading.
L2_EPS = 1e-6
#: default epsilon of RMSNormGated (the TKG page gives none; passed explicitly).
RMS_EPS = 1e-6


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------
def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits.  With x = m * 2**e, 0.5 <= |m| < 1,
    the result is round(m * 2**8) * 2**(e - 8) with numpy's half-to-even
    rounding.  Only the normal range is handled (no overflow or subnormals),
    which covers every value these tests produce.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def l2norm(x, eps=L2_EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis ("l2norm(q,k)", TKG page,
    summary line)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    """1 / (1 + exp(-x)) ("beta=sigmoid(b)", TKG page, summary line)."""
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def softplus(x):
    """log(1 + exp(x)), evaluated without overflow as logaddexp(0, x)
    ("softplus(a+dt_bias)", TKG page, summary line).  No threshold is applied."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def rms_norm_gated(o, z, weight, eps=RMS_EPS):
    """RMSNormGated(out, z) (TKG page, summary line; parameters z, norm_weight).

    Reading: normalise o by the root mean square over the value axis of one
    head, multiply by the weight (gamma) directly, then gate with silu(z):
        y = weight * o / sqrt(mean(o^2) + eps) * silu(z)
    """
    o = np.asarray(o, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return np.asarray(weight, np.float64) * (o / np.sqrt(ms + eps)) * silu(z)


# --------------------------------------------------------------------------
# prefill (GDN CTE Kernel API Reference, gdn_cte)
# --------------------------------------------------------------------------
def cte(query, key, value, g_log, beta, scale=1.0, initial_state=None):
    """Token-by-token gdn_cte.

    query, key: [B, Hk, S, Dk] (token-major, already unit length: the page's
    Notes require it and the oracle does not renormalise); value: [B, Hv, S, Dv];
    g_log, beta: [B, Hv, S]; initial_state: [B, Hv, Dk, Dv] or None (zero state,
    "parameter recurrent_state").  Value head h reads key/query head
    h // (Hv // Hk) (page Notes, GQA).

    Returns out [B, Hv, S, Dv] (un-normalised, "return" of gdn_cte) and the
    final state [B, Hv, Dk, Dv].

    Readings: the output uses the updated state S_t; the delta uses the decayed
    state (it follows from exp(g)(I - beta k k^T) S); scale multiplies q.
    """
    query = np.asarray(query, np.float64)
    key = np.asarray(key, np.float64)
    value = np.asarray(value, np.float64)
    g_log = np.asarray(g_log, np.float64)
    beta = np.asarray(beta, np.float64)
    B, Hk, S, Dk = query.shape
    Hv, Dv = value.shape[1], value.shape[3]
    assert Hv % Hk == 0
    kv_head = np.arange(Hv) // (Hv // Hk)

    if initial_state is None:
        St = np.zeros((B, Hv, Dk, Dv))
    else:
        St = np.array(initial_state, dtype=np.float64, copy=True)
    out = np.empty((B, Hv, S, Dv))
    for t in range(S):
        k = key[:, kv_head, t]                      # [B, Hv, Dk]
        q = query[:, kv_head, t]
        v = value[:, :, t]                          # [B, Hv, Dv]
        a = np.exp(g_log[:, :, t])[..., None, None]
        b = beta[:, :, t][..., None, None]
        # (I - b k k^T) S  ==  S - b k (k^T S)
        kS = np.einsum("bhk,bhkv->bhv", k, St)
        St = a * (St - b * k[..., :, None] * kS[..., None, :]) \
            + b * k[..., :, None] * v[..., None, :]
        out[:, :, t] = scale * np.einsum("bhkv,bhk->bhv", St, q)
    return out, St


# --------------------------------------------------------------------------
# decode step (GDN TKG Kernel API Reference, gdn_tkg)
# --------------------------------------------------------------------------
def cte_fused(q, k, v, b, a, A_log, dt_bias, z, norm_weight, initial_state=None, rms_eps=RMS_EPS):
    """gdn_cte with the decode step's gates before it and its output norm after
    it: the steps either side of the prefill ("GDN CTE Kernel API Reference",
    gdn_cte Notes: unit-length q, k; return: un-normalised output) in the form
    the "GDN TKG Kernel API Reference" summary gives them.

    q, k: [B, Hk, S, Dk] raw; v, z: [B, Hv, S, Dv]; b, a: [B, Hv, S];
    A_log, dt_bias: [Hv] (value head h); norm_weight: [Dv].
    q^ = l2norm(q), k^ = l2norm(k), beta = sigmoid(b),
    g = -exp(A_log[h]) softplus(a + dt_bias[h]);
    (O, S) = cte(q^, k^, v, g, beta, scale = Dk^-1/2, initial_state);
    y = RMSNormGated(O, z) per token over Dv.

    Returns (y [B, Hv, S, Dv] in float64, not rounded; S [B, Hv, Dk, Dv]).
    Reading: the scale is applied after the norm, as in the decode step; every
    intermediate is exact here (the device rounds q^, k^ and O to its type).
    """
    v = np.asarray(v, np.float64)
    Dk = np.asarray(q).shape[-1]
    q_unit, k_unit = l2norm(q), l2norm(k)
    beta_t = sigmoid(b)
    rate = np.exp(np.asarray(A_log, np.float64))[None, :, None]
    g = -rate * softplus(np.asarray(a, np.float64) + np.asarray(dt_bias, np.float64)[None, :, None])
    O, S = cte(q_unit, k_unit, v, g, beta_t, 1.0 / np.sqrt(Dk), initial_state)
    return rms_norm_gated(O, z, norm_weight, rms_eps), S


def tkg(q, k, v, b, a, A_log, dt_bias, z, norm_weight, state_in, num_v_heads,
        rms_eps=RMS_EPS):
    """One fused decode step for BH = B * num_v_heads independent heads.

    q, k: [BH, K] raw (not normalised); v, z: [BH, V]; b, a: [BH];
    A_log, dt_bias: [num_v_heads], indexed by bh % num_v_heads (heads cycle
    fastest per batch, page Dimensions); norm_weight: [V]; state_in [BH, K, V].

    Prologue (page summary and Notes): q^ = l2norm(q) / sqrt(K) (the 1/sqrt(K)
    query scale is applied after the norm), k^ = l2norm(k), beta = sigmoid(b),
    g = -exp(A_log) * softplus(a + dt_bias).  Core: one step of the recurrence,
    written here with the explicit transition matrix
    Phi = exp(g) (I - beta k^ k^T).  Epilogue: RMSNormGated(o, z), rounded to
    bf16 ("return": bf16 output).

    Returns (y [BH, V] as float64 holding bf16 values, state [BH, K, V]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S0 = np.asarray(state_in, np.float64)
    BH, K = q.shape
    head = np.arange(BH) % num_v_heads

    qn = l2norm(q) / np.sqrt(K)
    kn = l2norm(k)
    beta = sigmoid(b)
    g = -np.exp(np.asarray(A_log, np.float64)[head]) * softplus(
        np.asarray(a, np.float64) + np.asarray(dt_bias, np.float64)[head])

    eye = np.eye(K)
    Phi = np.exp(g)[:, None, None] * (
        eye - beta[:, None, None] * kn[:, :, None] * kn[:, None, :])
    S1 = Phi @ S0 + beta[:, None, None] * kn[:, :, None] * v[:, None, :]
    o = np.einsum("nkv,nk->nv", S1, qn)
    y = bf16_round(rms_norm_gated(o, z, norm_weight, rms_eps))
    return y, S1


# --------------------------------------------------------------------------
# fused decode layer (GDN Block TKG Kernel API Reference, gdn_block_tkg)
# --------------------------------------------------------------------------
def in_proj(hidden, W):
    """hidden [B, H] times W [H, N] (W == nn.Linear.weight.T, page parameters),
    accumulated exactly in float64 and rounded to bf16 (reading: bf16
    activations at every stage boundary)."""
    return bf16_round(np.asarray(hidden, np.float64) @ np.asarray(W, np.float64))


def conv1d_decode(x_new, conv_state, conv_weight):
    """Depthwise causal conv1d decode ("conv + silu + slide-window state",
    Block TKG page summary).

    x_new [B, C] (bf16 values), conv_state [B, C, K_win] (bf16 values, oldest
    first), conv_weight [C, K_win].  Reading: the window drops its oldest
    slot and appends the new input; tap K_win-1 multiplies the newest input;
    no bias.  Returns (silu(sum_j w[c,j] * window[b,c,j]) in float64,
    new window).
    """
    window = np.concatenate(
        [np.asarray(conv_state, np.float64)[:, :, 1:],
         np.asarray(x_new, np.float64)[:, :, None]], axis=2)
    acc = np.sum(window * np.asarray(conv_weight, np.float64)[None], axis=2)
    return silu(acc), window


def block_tkg(hidden, W_in_qkv, W_in_z, W_in_a, W_in_b, conv_weight, conv_state,
              A_log, dt_bias, norm_weight, recurrent_state, num_k_heads,
              num_v_heads, head_k_dim, head_v_dim, rms_eps=RMS_EPS):
    """gdn_block_tkg: in_proj -> conv1d decode -> split q|k|v + GQA repeat ->
    gdn_tkg -> [B, 1, value_dim].  Functional (page Notes): returns
    (out, conv_state', recurrent_state').

    Readings: q|k|v are packed as contiguous blocks [q (key_dim) | k (key_dim) |
    v (value_dim)]; the conv output is rounded to bf16 before the decode step
    (the bf16 window stores the same stage's input); a and b are the bf16
    projections widened for the gate math; the output is bf16.
    """
    hidden = np.asarray(hidden, np.float64)
    B = hidden.shape[0]
    x = hidden.reshape(B, -1)
    Hk, Hv, Dk, Dv = num_k_heads, num_v_heads, head_k_dim, head_v_dim
    key_dim = Hk * Dk

    mixed = in_proj(x, W_in_qkv)
    zz = in_proj(x, W_in_z)
    aa = in_proj(x, W_in_a)
    bb = in_proj(x, W_in_b)
    conv_out, new_window = conv1d_decode(mixed, conv_state, conv_weight)
    conv_out = bf16_round(conv_out)

    q = conv_out[:, :key_dim].reshape(B, Hk, Dk)
    k = conv_out[:, key_dim:2 * key_dim].reshape(B, Hk, Dk)
    v = conv_out[:, 2 * key_dim:].reshape(B, Hv, Dv)
    kv_head = np.arange(Hv) // (Hv // Hk)
    q = q[:, kv_head].reshape(B * Hv, Dk)
    k = k[:, kv_head].reshape(B * Hv, Dk)

    y, S1 = tkg(q, k, v.reshape(B * Hv, Dv), bb.reshape(B * Hv), aa.reshape(B * Hv),
                A_log, dt_bias, zz.reshape(B * Hv, Dv), norm_weight,
                np.asarray(recurrent_state, np.float64).reshape(B * Hv, Dk, Dv),
                Hv, rms_eps)
    return y.reshape(B, 1, Hv * Dv), new_window, S1.reshape(B, Hv, Dk, Dv)


# --------------------------------------------------------------------------
# prefill counterpart of the decode layer: in_proj over S tokens, the causal
# conv1d over the sequence, then the prefill with the decode gates and norm
# --------------------------------------------------------------------------
def conv1d_prefill(x, conv_state, conv_weight):
    """The decode conv1d applied along a sequence ("conv + silu + slide-window
    state", Block TKG page summary, read for S tokens at once).

    x [B, S, C] (bf16 values), conv_state [B, C, K_win] (oldest first),
    conv_weight [C, K_win].  Per channel the inputs extend the window:
    e = [conv_state[..., 0], ..., conv_state[..., K_win-1], x_0, ..., x_{S-1}];
    token t sees e[t+1 .. t+K_win] (tap K_win-1 on x_t) and the returned window
    is the last K_win entries of e.  Returns (silu(conv) [B, S, C] in float64,
    new window [B, C, K_win]).
    """
    x = np.asarray(x, np.float64)
    B, S, C = x.shape
    st = np.asarray(conv_state, np.float64)
    Kw = st.shape[2]
    e = np.concatenate([st, np.transpose(x, (0, 2, 1))], axis=2)       # [B, C, K_win + S]
    w = np.asarray(conv_weight, np.float64)
    acc = np.zeros((B, C, S))
    for j in range(Kw):
        acc += w[None, :, j:j + 1] * e[:, :, 1 + j:1 + j + S]
    return np.transpose(silu(acc), (0, 2, 1)), e[:, :, S:S + Kw]


def block_cte(hidden, W_in_qkv, W_in_z, W_in_a, W_in_b, conv_weight, conv_state,
              A_log, dt_bias, norm_weight, recurrent_state, num_k_heads,
              num_v_heads, head_k_dim, head_v_dim, rms_eps=RMS_EPS):
    """Prefill layer: hidden [B, S, H] -> in_proj (bf16 stage outputs) -> conv1d
    over the sequence (bf16 output) -> split q|k|v (contiguous blocks) ->
    cte_fused (per-head q, k; GQA by h // (Hv / Hk)) -> [B, S, value_dim].

    Returns (out [B, S, value_dim] in float64, not rounded; conv_state'
    [B, conv_dim, K_win]; recurrent_state' [B, Hv, Dk, Dv]).  The same
    readings as block_tkg; the output is left unrounded.
    """
    hidden = np.asarray(hidden, np.float64)
    B, S, H = hidden.shape
    Hk, Hv, Dk, Dv = num_k_heads, num_v_heads, head_k_dim, head_v_dim
    key_dim = Hk * Dk
    x = hidden.reshape(B * S, H)
    mixed = in_proj(x, W_in_qkv).reshape(B, S, -1)
    zz = in_proj(x, W_in_z).reshape(B, S, Hv, Dv)
    aa = in_proj(x, W_in_a).reshape(B, S, Hv)
    bb = in_proj(x, W_in_b).reshape(B, S, Hv)
    conv_out, new_window = conv1d_prefill(mixed, conv_state, conv_weight)
    conv_out = bf16_round(conv_out)
    q = conv_out[:, :, :key_dim].reshape(B, S, Hk, Dk).transpose(0, 2, 1, 3)
    k = conv_out[:, :, key_dim:2 * key_dim].reshape(B, S, Hk, Dk).transpose(0, 2, 1, 3)
    v = conv_out[:, :, 2 * key_dim:].reshape(B, S, Hv, Dv).transpose(0, 2, 1, 3)
    y, S1 = cte_fused(q, k, v, bb.transpose(0, 2, 1), aa.transpose(0, 2, 1), A_log, dt_bias,
                      zz.transpose(0, 2, 1, 3), norm_weight, recurrent_state, rms_eps)
    return y.transpose(0, 2, 1, 3).reshape(B, S, Hv * Dv), new_window, S1
