"""The oracle pins have teeth: each plausible mistake planted in a copy of the
oracle's source (CPU only) must make at least one pin fail."""
import types

import pytest

import tests.test_oracle_pins as pins
from oracle import gdn_ref

with open(gdn_ref.__file__) as _f:
    SRC = _f.read()

# (label, exact source text, replacement)
MUTANTS = [
    ("decay sign", "a = np.exp(g_log[:, :, t])", "a = np.exp(-g_log[:, :, t])"),
    ("delta sign", "St = a * (St - b * k", "St = a * (St + b * k"),
    ("undecayed delta", "St = a * (St - b * k[..., :, None] * kS[..., None, :])",
     "St = a * St - b * k[..., :, None] * kS[..., None, :]"),
    ("delta uses q", 'kS = np.einsum("bhk,bhkv->bhv", k, St)', 'kS = np.einsum("bhk,bhkv->bhv", q, St)'),
    ("write without beta", "+ b * k[..., :, None] * v[..., None, :]", "+ k[..., :, None] * v[..., None, :]"),
    ("GQA map", "kv_head = np.arange(Hv) // (Hv // Hk)\n\n    if", "kv_head = np.arange(Hv) % Hk\n\n    if"),
    ("dropped scale", "out[:, :, t] = scale * np.einsum", "out[:, :, t] = np.einsum"),
    ("output from old state", 'out[:, :, t] = scale * np.einsum("bhkv,bhk->bhv", St, q)',
     'out[:, :, t] = scale * np.einsum("bhkv,bhk->bhv", St, k)'),
    ("no query scale in decode", "qn = l2norm(q) / np.sqrt(K)", "qn = l2norm(q)"),
    ("gate sign", "g = -np.exp(np.asarray(A_log", "g = np.exp(np.asarray(A_log"),
    ("head index", "head = np.arange(BH) % num_v_heads", "head = np.arange(BH) // num_v_heads"),
    ("no softplus", "* softplus(\n", "* (\n"),
    ("beta not sigmoid", "    beta = sigmoid(b)\n", "    beta = np.asarray(b, np.float64)\n"),
    ("rms sum not mean", "ms = np.mean(o * o, axis=-1, keepdims=True)", "ms = np.sum(o * o, axis=-1, keepdims=True)"),
    ("gate sigmoid not silu", "* (o / np.sqrt(ms + eps)) * silu(z)", "* (o / np.sqrt(ms + eps)) * sigmoid(z)"),
    ("transposed state operand", "S1 = Phi @ S0", "S1 = Phi @ np.swapaxes(S0, 1, 2)"),
    ("k from q block", "k = conv_out[:, key_dim:2 * key_dim]", "k = conv_out[:, :key_dim]"),
    ("window order", "np.asarray(conv_state, np.float64)[:, :, 1:]", "np.asarray(conv_state, np.float64)[:, :, :-1]"),
    ("bf16 ties away", "np.round(np.ldexp(m, 8))", "np.floor(np.ldexp(m, 8) + 0.5)"),
    ("sequence conv tap offset", "acc += w[None, :, j:j + 1] * e[:, :, 1 + j:1 + j + S]",
     "acc += w[None, :, j:j + 1] * e[:, :, j:j + S]"),
    ("sequence conv window end", "e[:, :, S:S + Kw]", "e[:, :, S - 1:S - 1 + Kw]"),
    ("prefill layer k from q block", "k = conv_out[:, :, key_dim:2 * key_dim]", "k = conv_out[:, :, :key_dim]"),
    ("fused gate head order", "rate = np.exp(np.asarray(A_log, np.float64))[None, :, None]",
     "rate = np.exp(np.asarray(A_log, np.float64))[::-1][None, :, None]"),
    ("fused beta not sigmoid", "beta_t = sigmoid(b)", "beta_t = np.asarray(b, np.float64)"),
    ("fused key not normalised", "q_unit, k_unit = l2norm(q), l2norm(k)", "q_unit, k_unit = l2norm(q), k"),
    ("fused output rescaled", "return rms_norm_gated(O, z, norm_weight, rms_eps), S",
     "return rms_norm_gated(O, z, norm_weight, rms_eps) * 1.01, S"),
]

CHECKS = [
    (pins.test_cte_hand_worked_example, dict(impl="numpy")),
    (pins.test_cte_mpmath_bruteforce, dict(impl="numpy", Dk=2, Dv=3, S=4)),
    (pins.test_cte_beta_zero_is_pure_decay, dict(impl="numpy")),
    (pins.test_cte_write_is_exact_for_orthonormal_keys, dict(impl="numpy")),
    (pins.test_cte_scalar_geometric_closed_form, dict(impl="numpy")),
    (pins.test_cte_gqa_equals_explicit_repeat, dict(impl="numpy")),
    (pins.test_cte_single_chunk_wy_form_via_triangular_solve, dict(impl="numpy", S=17)),
    (pins.test_cte_c_twin_matches_numpy, {}),
    (pins.test_bf16_round_known_values_and_generator_agreement, {}),
    (pins.test_tkg_hand_worked_example, dict(impl="numpy")),
    (pins.test_tkg_gate_and_head_indexing, dict(impl="numpy")),
    (pins.test_tkg_constant_output_closed_form, dict(impl="numpy")),
    (pins.test_rms_norm_gated_properties, {}),
    (pins.test_tkg_c_twin_matches_numpy, {}),
    (pins.test_conv1d_decode_one_hot_and_correlate, {}),
    (pins.test_conv1d_decode_window_after_k_steps_holds_last_inputs, {}),
    (pins.test_block_wiring_split_and_gqa, {}),
    (pins.test_cte_fused_equals_iterated_decode_steps, dict(Hk=1, Hv=3)),
    (pins.test_conv1d_prefill_equals_decode_conv_token_by_token, {}),
    (pins.test_block_cte_equals_iterated_decode_layer, dict(Hk=1, Hv=2)),
]


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("gdn_ref_mutant")
    exec(compile(SRC.replace(old, new), "gdn_ref_mutant.py", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes_all_checks(monkeypatch):
    mod = _mutant("__all__", "__all__")
    monkeypatch.setattr(pins, "gdn_ref", mod)
    monkeypatch.setitem(pins.CTE_IMPLS, "numpy", mod.cte)
    monkeypatch.setitem(pins.TKG_IMPLS, "numpy", mod.tkg)
    for fn, kw in CHECKS:
        fn(**kw)


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(label, old, new, monkeypatch):
    mod = _mutant(old, new)
    monkeypatch.setattr(pins, "gdn_ref", mod)
    monkeypatch.setitem(pins.CTE_IMPLS, "numpy", mod.cte)
    monkeypatch.setitem(pins.TKG_IMPLS, "numpy", mod.tkg)
    caught = []
    for fn, kw in CHECKS:
        try:
            fn(**kw)
        except Exception as e:  # an assertion or a shape error both expose the mistake
            caught.append((fn.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {label!r}"
