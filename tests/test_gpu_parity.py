"""GPU parity: every libgdn entry point, called through the C ABI (via the thin
binding), against the fp64 CPU oracle on the same seeded inputs."""
import math

import numpy as np
import pytest

from gated_delta_rule_cte_amd import inputs
from oracle import c_ref, gdn_ref
from tests.gpu_util import TOL_BF16, TOL_F32, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def _run_cte(gdn, d, with_state, algorithm=0):
    st = dev(d["recurrent_state"]).clone() if with_state else None
    out, state = gdn.gdn_cte(dev(d["query"]), dev(d["key"]), dev(d["value"]), dev(d["g_log"]),
                             dev(d["beta"]), d["scale"], recurrent_state=st, algorithm=algorithm)
    _sync()
    return host(out), host(state)


def _oracle_cte(d, with_state, heads=None):
    """C-twin oracle; `heads` = list of (b, h) to evaluate (None = all)."""
    q, k, v = d["query"].f64(), d["key"].f64(), d["value"].f64()
    g, be = d["g_log"].f64(), d["beta"].f64()
    s0 = d["recurrent_state"].f64() if with_state else None
    if heads is None:
        return c_ref.cte(q, k, v, g, be, d["scale"], s0)
    # gather the sampled heads into one batch-1 call (key head per value head)
    Hk, Hv = q.shape[1], v.shape[1]
    kv = [h // (Hv // Hk) for _, h in heads]
    bs = [b for b, _ in heads]
    hs = [h for _, h in heads]
    ro, rs = c_ref.cte(q[bs, kv][None], k[bs, kv][None], v[bs, hs][None], g[bs, hs][None],
                       be[bs, hs][None], d["scale"], None if s0 is None else s0[bs, hs][None])
    return {bh: (ro[:, i:i + 1], rs[:, i:i + 1]) for i, bh in enumerate(heads)}


CTE_CASES = [
    # (B, Hk, Hv, S, Dk, Dv, dtype, with_state)
    (1, 2, 2, 128, 64, 64, "f32", False),      # the small fp32 workload's shape
    (2, 1, 3, 77, 64, 32, "f32", True),        # ragged tail, GQA 1:3, narrow Dv
    (1, 2, 4, 200, 128, 128, "f32", True),     # DK = 128 fp32 path, several chunks
    (1, 1, 1, 1, 16, 24, "f32", True),         # one token, tiny odd dims
    (1, 2, 4, 300, 128, 128, "bf16", True),    # ragged, GQA 1:2, in-place state
    (2, 2, 2, 64, 40, 72, "bf16", False),      # padded Dk, Dv not a tile multiple
    (1, 4, 4, 1000, 64, 128, "bf16", True),    # DK = 64 bf16 path
    (1, 1, 2, 2373, 64, 64, "bf16", True),     # 38 chunks, ragged tail
    (1, 1, 1, 1100, 128, 48, "bf16", False),   # 18 chunks (odd chunk-pair count), one value head per key head
    (1, 1, 3, 300, 64, 64, "bf16", True),      # GQA 1:3 (odd group: one value head per chunk-local wave)
    (2, 2, 4, 333, 64, 64, "bf16", True),      # GQA 1:2 with DK = 64 (value-head pairs per wave)
]


@pytest.mark.parametrize("case", CTE_CASES, ids=lambda c: "B{}_Hk{}_Hv{}_S{}_Dk{}_Dv{}_{}_{}".format(
    *c[:7], "state" if c[7] else "zero"))
def test_cte_matches_oracle(gpu_lib, case):
    B, Hk, Hv, S, Dk, Dv, dt, ws = case
    d = inputs.cte_inputs(B, Hk, Hv, S, Dk, Dv, dtype=dt, g_range=(-0.5, -0.01),
                          state_std=0.05 if ws else None, seed=1000 + S)
    o, s = _run_cte(gpu_lib, d, ws)
    ro, rs = _oracle_cte(d, ws)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(o, ro, tol, 2, "out")
    assert_close(s, rs, tol, 2, "state")


NEUMANN_CASES = [CTE_CASES[i] for i in (0, 1, 2, 4, 6, 8, 9, 10)]


@pytest.mark.parametrize("case", NEUMANN_CASES, ids=lambda c: "B{}_Hk{}_Hv{}_S{}_Dk{}_Dv{}_{}_{}".format(
    *c[:7], "state" if c[7] else "zero"))
def test_cte_neumann_inverse_matches_oracle(gpu_lib, case):
    """GDN_CTE_ALGO_NEUMANN (the intra-chunk inverse as the doubling Neumann product)
    against the same oracle and tolerances as the default method."""
    B, Hk, Hv, S, Dk, Dv, dt, ws = case
    d = inputs.cte_inputs(B, Hk, Hv, S, Dk, Dv, dtype=dt, g_range=(-0.5, -0.01),
                          state_std=0.05 if ws else None, seed=1000 + S)
    o, s = _run_cte(gpu_lib, d, ws, algorithm=gpu_lib.GDN_CTE_ALGO_NEUMANN)
    ro, rs = _oracle_cte(d, ws)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(o, ro, tol, 2, "out")
    assert_close(s, rs, tol, 2, "state")


def test_cte_neumann_s4096_workload_close_to_default(gpu_lib):
    """At the S=4096 GQA workload both inverse methods meet the oracle bar, and they
    agree with each other far inside it (they differ only in T's fp32 rounding)."""
    d = inputs.workload_inputs("cte_bf16_b1_hk16_hv32_s4096_d128")
    o0, s0 = _run_cte(gpu_lib, d, True)
    o1, s1 = _run_cte(gpu_lib, d, True, algorithm=gpu_lib.GDN_CTE_ALGO_NEUMANN)
    heads = [(0, h) for h in (0, 7, 18, 31)]
    ref = _oracle_cte(d, True, heads)
    for (b, h), (ro, rs) in ref.items():
        assert_close(o1[b:b + 1, h:h + 1], ro, TOL_BF16, 2, f"out head {h}")
        assert_close(s1[b:b + 1, h:h + 1], rs, TOL_BF16, 2, f"state head {h}")
    assert_close(o1, o0.astype(np.float64), 2e-3, 2, "out vs default")
    assert_close(s1, s0.astype(np.float64), 2e-3, 2, "state vs default")


FUSED_CASES = [
    # (B, Hk, Hv, S, Dk, Dv, dtype, with_state)
    (1, 2, 2, 128, 64, 64, "f32", True),
    (2, 1, 3, 77, 64, 32, "f32", False),
    (1, 2, 4, 300, 128, 128, "bf16", True),
    (1, 1, 1, 1100, 128, 48, "bf16", False),
    (2, 2, 4, 333, 64, 64, "bf16", True),
    # several chunk-local waves per key head: one of them writes the unit q, k rows
    (1, 1, 4, 200, 128, 64, "bf16", True),
    (1, 2, 6, 150, 64, 64, "bf16", False),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "B{}_Hk{}_Hv{}_S{}_Dk{}_Dv{}_{}_{}".format(
    *c[:7], "state" if c[7] else "zero"))
@pytest.mark.parametrize("algorithm", [0, 1])
def test_cte_fused_matches_oracle(gpu_lib, case, algorithm):
    """gdn_cte_fused (raw q, k; decode gates; RMSNormGated output) against the
    oracle's composition of the same steps."""
    B, Hk, Hv, S, Dk, Dv, dt, ws = case
    d = inputs.cte_fused_inputs(B, Hk, Hv, S, Dk, Dv, dtype=dt, state_std=0.05 if ws else None, seed=2000 + S)
    st = dev(d["recurrent_state"]).clone() if ws else None
    y, state = gpu_lib.gdn_cte_fused(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["b"]), dev(d["a"]),
                                     dev(d["A_log"]), dev(d["dt_bias"]), dev(d["z"]), dev(d["norm_weight"]),
                                     recurrent_state=st, algorithm=algorithm)
    _sync()
    ry, rs = gdn_ref.cte_fused(d["q"].f64(), d["k"].f64(), d["v"].f64(), d["b"].f64(), d["a"].f64(),
                               d["A_log"].f64(), d["dt_bias"].f64(), d["z"].f64(), d["norm_weight"].f64(),
                               d["recurrent_state"].f64() if ws else None)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(host(y), ry, tol, 2, "out")
    assert_close(host(state), rs, tol, 2, "state")


BLOCK_CTE_CASES = [
    # (B, S, H, Hk, Hv, Dk, Dv, K_win, in_place, algorithm)
    (2, 100, 128, 2, 4, 32, 32, 4, False, 0),
    (1, 300, 256, 1, 2, 64, 64, 3, True, 0),
    (1, 2, 128, 2, 2, 16, 24, 4, True, 0),      # fewer tokens than the conv window
    (1, 130, 128, 2, 2, 128, 128, 4, False, 1),  # full head dims, Neumann inverse
    (2, 70, 256, 4, 8, 32, 32, 4, True, 0),      # Hv % 8 == 0: a and b on the GEMM
    # Hv % 16 == 0: a and b on their MFMA kernel (16, 48, 64 columns; token
    # rows not a multiple of 16; H = 384 gives each wave three k-steps)
    (2, 37, 256, 4, 16, 32, 32, 4, False, 0),
    (1, 45, 128, 8, 48, 16, 16, 4, True, 0),
    (3, 21, 384, 16, 64, 16, 16, 4, False, 0),
    (1, 3, 128, 2, 16, 16, 16, 2, True, 0),     # fewer token rows than one 16-row tile
    # GQA groups of 3 and 4: the q, k rows are normalised by a separate pass
    # (several chunk-local waves read each key head, so none may overwrite it)
    (1, 90, 128, 1, 3, 32, 32, 4, False, 0),
    (1, 70, 128, 1, 4, 32, 32, 4, True, 1),
    # the longest conv windows the API accepts, one of them longer than the sequence
    (1, 50, 128, 2, 4, 32, 32, 8, True, 0),
    (2, 37, 128, 1, 2, 32, 32, 5, False, 0),
    (1, 5, 128, 1, 1, 16, 16, 8, True, 0),
]


@pytest.mark.parametrize("case", BLOCK_CTE_CASES, ids=lambda c: "B{}_S{}_H{}_Hk{}_Hv{}_Dk{}_Dv{}_W{}_{}_a{}".format(
    *c[:8], "inplace" if c[8] else "copy", c[9]))
def test_block_cte_matches_oracle(gpu_lib, case):
    """gdn_block_cte (in_proj GEMMs, the conv over the sequence, the fused prefill)
    against the oracle's prefill layer."""
    import torch
    B, S, H, Hk, Hv, Dk, Dv, W, in_place, algo = case
    d = inputs.block_cte_inputs(B, S, H, Hk, Hv, Dk, Dv, K_win=W, seed=3000 + S)
    cs = dev(d["conv_state"]).clone()
    rs = dev(d["recurrent_state"]).clone()
    args = [dev(d[n]) for n in ("hidden", "W_in_qkv", "W_in_z", "W_in_a", "W_in_b", "conv_weight")]
    out, cs1, rs1 = gpu_lib.gdn_block_cte(*args, cs, dev(d["A_log"]), dev(d["dt_bias"]), dev(d["norm_weight"]), rs,
                                          algorithm=algo, conv_state_out=cs if in_place else None,
                                          recurrent_state_out=rs if in_place else None)
    _sync()
    ry, rcs, rrs = gdn_ref.block_cte(d["hidden"].f64(), d["W_in_qkv"].f64(), d["W_in_z"].f64(), d["W_in_a"].f64(),
                                     d["W_in_b"].f64(), d["conv_weight"].f64(), d["conv_state"].f64(),
                                     d["A_log"].f64(), d["dt_bias"].f64(), d["norm_weight"].f64(),
                                     d["recurrent_state"].f64(), Hk, Hv, Dk, Dv)
    assert_close(host(out), ry, TOL_BF16, 1, "out")
    assert_close(host(rs1), rrs, TOL_BF16, 2, "recurrent state")
    # the final window: entries carried over from the old window are copied bit
    # for bit, the others are the bf16-rounded projections of the last tokens
    win, n_new = host(cs1), min(S, W)
    np.testing.assert_array_equal(win[..., :W - n_new], rcs[..., :W - n_new])
    assert_bf16_sums_match(win[..., W - n_new:], rcs[..., W - n_new:], d["hidden"].f64()[:, S - n_new:],
                           d["W_in_qkv"].f64(), "conv window")
    if in_place:
        assert cs1.data_ptr() == cs.data_ptr() and rs1.data_ptr() == rs.data_ptr()


def test_block_cte_one_token_equals_decode_layer(gpu_lib):
    """One token through the prefill layer and through gdn_block_tkg: the same
    caches and outputs within the bf16 bar.  The slid part of the conv window
    is the input window's in both, bit for bit; its new column is each path's
    bf16 rounding of an fp32 sum of hidden @ W_qkv, and the two paths sum in
    different orders (the prefill layer's projection runs on the vendor GEMM
    library), so each is held to the rounding interval of the exact sum."""
    d = inputs.block_cte_inputs(3, 1, 256, 2, 4, 64, 64, K_win=4, seed=33)
    names = ("hidden", "W_in_qkv", "W_in_z", "W_in_a", "W_in_b", "conv_weight")
    args = [dev(d[n]) for n in names]
    rest = [dev(d[n]) for n in ("conv_state", "A_log", "dt_bias", "norm_weight", "recurrent_state")]
    out, cs1, rs1 = gpu_lib.gdn_block_cte(*args, *rest)
    out2, cs2, rs2 = gpu_lib.gdn_block_tkg(*args, *rest)
    _sync()
    c1, c2 = host(cs1), host(cs2)
    np.testing.assert_array_equal(c1[..., :-1], c2[..., :-1])
    hid, wq = d["hidden"].f64(), d["W_in_qkv"].f64()
    ref = gdn_ref.bf16_round(np.matmul(hid, wq)).transpose(0, 2, 1)
    assert_bf16_sums_match(c1[..., -1:], ref, hid, wq, "conv window's new column (prefill layer)")
    assert_bf16_sums_match(c2[..., -1:], ref, hid, wq, "conv window's new column (decode layer)")
    assert_close(host(out), host(out2), TOL_BF16, 1, "out")
    assert_close(host(rs1), host(rs2), TOL_BF16, 2, "recurrent state")


def test_cte_empty_sequence(gpu_lib):
    import torch
    d = inputs.cte_inputs(1, 2, 2, 0, 64, 64, dtype="bf16", state_std=0.05, seed=5)
    init = dev(d["recurrent_state"]).clone()
    out, st = gpu_lib.gdn_cte(dev(d["query"]), dev(d["key"]), dev(d["value"]), dev(d["g_log"]),
                              dev(d["beta"]), d["scale"], recurrent_state=init.clone())
    _sync()
    assert out.shape == (1, 2, 0, 64)
    assert torch.equal(st, init)
    out, st = gpu_lib.gdn_cte(dev(d["query"]), dev(d["key"]), dev(d["value"]), dev(d["g_log"]),
                              dev(d["beta"]), d["scale"])
    _sync()
    assert torch.count_nonzero(st).item() == 0


def test_cte_small_fp32_workload(gpu_lib):
    """B=1, Hk=Hv=2, S=128, Dk=Dv=64, fp32, zero state: element-by-element."""
    d = inputs.workload_inputs("cte_fp32_b1_h2_s128_d64")
    o, s = _run_cte(gpu_lib, d, False)
    ro, rs = gdn_ref.cte(d["query"].f64(), d["key"].f64(), d["value"].f64(), d["g_log"].f64(),
                         d["beta"].f64(), d["scale"], None)
    assert_close(o, ro, TOL_F32, 2, "out")
    assert_close(s, rs, TOL_F32, 2, "state")


def test_cte_gqa_s4096_workload(gpu_lib):
    """B=1, Hk=16, Hv=32, S=4096, D=128, bf16, supplied state updated in place:
    every head against the oracle."""
    d = inputs.workload_inputs("cte_bf16_b1_hk16_hv32_s4096_d128")
    o, s = _run_cte(gpu_lib, d, True)
    ro, rs = _oracle_cte(d, True)
    assert_close(o, ro, TOL_BF16, 2, "out")
    assert_close(s, rs, TOL_BF16, 2, "state")


def test_cte_long_batched_workload_and_chaining(gpu_lib):
    """B=4, Hk=16, Hv=32, S=16384, D=128, bf16, zero state: all 128 (batch, value
    head) slices of the output and the final state against the oracle; four
    chained S=4096 calls carrying the state equal the single call bit for bit."""
    import torch
    d = inputs.workload_inputs("cte_bf16_b4_hk16_hv32_s16384_d128")
    q, k, v = dev(d["query"]), dev(d["key"]), dev(d["value"])
    g, be = dev(d["g_log"]), dev(d["beta"])
    out, st = gpu_lib.gdn_cte(q, k, v, g, be, d["scale"])
    _sync()
    ro, rs = _oracle_cte(d, False)
    assert_close(host(out), ro, TOL_BF16, 2, "out")
    assert_close(host(st), rs, TOL_BF16, 2, "state")
    del ro, rs
    # chained: 4 x 4096 with the state carried
    state = None
    outs = []
    for c in range(4):
        sl = slice(4096 * c, 4096 * (c + 1))
        oc, state = gpu_lib.gdn_cte(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(),
                                    v[:, :, sl].contiguous(), g[:, :, sl].contiguous(),
                                    be[:, :, sl].contiguous(), d["scale"], recurrent_state=state)
        outs.append(oc)
    _sync()
    assert torch.equal(torch.cat(outs, dim=2), out), "chained outputs differ from the single call"
    assert torch.equal(state, st), "chained final state differs from the single call"


def test_cte_inside_graph_capture(gpu_lib):
    """The prefill (chunk-local kernel, then the state pass, on the caller's
    stream) captured in a HIP graph: every replay, with eager work and syncs
    between replays, equals the eager call bit for bit."""
    import torch
    d = inputs.cte_inputs(1, 2, 4, 2048 + 64 * 5 + 17, 128, 128, dtype="bf16", state_std=0.05, seed=91)
    q, k, v, g, be = (dev(d[n]) for n in ("query", "key", "value", "g_log", "beta"))
    s0 = dev(d["recurrent_state"])
    st = s0.clone()
    out = torch.empty((1, 4, q.shape[2], 128), dtype=torch.bfloat16, device=q.device)
    gpu_lib.gdn_cte(q, k, v, g, be, d["scale"], recurrent_state=st, out=out)  # eager
    _sync()
    ref_out, ref_st = out.clone(), st.clone()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        st.copy_(s0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            gpu_lib.gdn_cte(q, k, v, g, be, d["scale"], recurrent_state=st, out=out)
    for _ in range(3):
        out.zero_()
        st.copy_(s0)
        _sync()
        graph.replay()
        _sync()
        assert torch.equal(out, ref_out), "graph replay output differs from the eager call"
        assert torch.equal(st, ref_st), "graph replay state differs from the eager call"


def test_cte_is_deterministic(gpu_lib):
    import torch
    d = inputs.cte_inputs(1, 2, 4, 500, 128, 128, dtype="bf16", state_std=0.05, seed=77)
    a = _run_cte(gpu_lib, d, True)
    b = _run_cte(gpu_lib, d, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_cte_beta_zero_is_pure_decay(gpu_lib, dt):
    """beta = 0: nothing is written, so S_t = exp(gam_t) S0 and
    o_t = scale exp(gam_t) S0^T q_t (gam = inclusive cumsum of g_log), for the
    outputs of every token and the final state."""
    d = inputs.cte_inputs(1, 2, 4, 300, 128, 128 if dt == "bf16" else 64, dtype=dt, state_std=0.05, seed=78)
    d["beta"] = inputs.f32(np.zeros_like(d["beta"].data))
    o, s = _run_cte(gpu_lib, d, True)
    gam = np.cumsum(d["g_log"].f64(), axis=-1)                       # [B, Hv, S]
    S0 = d["recurrent_state"].f64()                                  # [B, Hv, Dk, Dv]
    G = d["value"].shape[1] // d["query"].shape[1]
    qv = np.repeat(d["query"].f64(), G, axis=1)                      # [B, Hv, S, Dk]
    ref_o = d["scale"] * np.exp(gam)[..., None] * np.einsum("bhsk,bhkv->bhsv", qv, S0)
    ref_s = np.exp(gam[..., -1])[..., None, None] * S0
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(o, ref_o, tol, 2, "pure-decay outputs")
    assert_close(s, ref_s, tol, 2, "pure-decay state")


def _orthonormal_keys_case(dtype, n, Dk, Dv, seed):
    """g = 0, beta = 1, q_t = k_t, keys k_0..k_{n-1} orthonormal: fp32 keys
    are rows of a random orthogonal matrix; bf16 keys are signed unit
    vectors (exact in bf16)."""
    rng = np.random.default_rng(seed)
    if dtype == "f32":
        Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
        keys = Qm[:n]
    else:
        keys = np.zeros((n, Dk))
        keys[np.arange(n), rng.permutation(Dk)[:n]] = rng.choice([-1.0, 1.0], n)
    d = inputs.cte_inputs(1, 1, 1, n, Dk, Dv, dtype=dtype, state_std=0.05, seed=seed)
    kq = inputs.cast(keys[None, None], dtype)
    d["query"], d["key"] = kq, kq
    d["g_log"] = inputs.f32(np.zeros((1, 1, n)))
    d["beta"] = inputs.f32(np.ones((1, 1, n)))
    return d, keys


@pytest.mark.parametrize("dt,n", [("f32", 100), ("bf16", 100), ("bf16", 128)])
def test_cte_write_exact_with_orthonormal_keys(gpu_lib, dt, n):
    """With g = 0 and beta = 1 the rule writes v exactly: after the call
    S^T k_j = v_j for every written key, o_t = scale v_t (q_t = k_t), and
    directions orthogonal to every written key keep S0's response."""
    Dk, Dv = 128, 64 if dt == "f32" else 128
    d, keys = _orthonormal_keys_case(dt, n, Dk, Dv, seed=80 + n)
    o, s = _run_cte(gpu_lib, d, True)
    kf = d["key"].f64()[0, 0]                                        # the keys the device read
    v = d["value"].f64()[0, 0]
    S0 = d["recurrent_state"].f64()[0, 0]
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(o[0, 0], d["scale"] * v, tol, 0, "outputs = scale v")
    assert_close(kf @ s[0, 0], v, tol, 0, "S^T k_j = v_j")
    if n < Dk:
        # an orthonormal basis of the complement of the written keys
        u = np.linalg.svd(kf, full_matrices=True)[2][n:]
        assert_close(u @ s[0, 0], u @ S0, tol, 0, "orthogonal directions keep S0")


def test_cte_zero_state_never_reads_the_buffer(gpu_lib):
    """has_initial_state = 0 through the C ABI with the state buffer filled with
    NaN: the state is never read (the outputs and final state are finite and
    equal, bit for bit, those of a call whose buffer holds zeros)."""
    import ctypes
    import torch
    for dt, Dk in (("bf16", 128), ("f32", 64)):
        d = inputs.cte_inputs(1, 2, 4, 333, Dk, Dk, dtype=dt, seed=79)
        q, k, v, g, be = (dev(d[n]) for n in ("query", "key", "value", "g_log", "beta"))
        B, Hk, S, _ = q.shape
        Hv = v.shape[1]
        lib = gpu_lib.load()
        code = gpu_lib.GDN_BF16 if dt == "bf16" else gpu_lib.GDN_F32
        ws_bytes = lib.gdn_cte_workspace_size(B, Hk, Hv, S, Dk, Dk, code)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
        res = []
        for fill in (float("nan"), 0.0):
            st = torch.full((B, Hv, Dk, Dk), fill, dtype=torch.float32, device=q.device)
            out = torch.empty_like(v)
            stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            rc = lib.gdn_cte(*(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, g, be)), d["scale"],
                             ctypes.c_void_p(st.data_ptr()), 0, ctypes.c_void_p(out.data_ptr()),
                             B, Hk, Hv, S, Dk, Dk, code, 0, ctypes.c_void_p(ws.data_ptr()), ws_bytes, stream)
            assert rc == 0, lib.gdn_last_error().decode()
            _sync()
            res.append((out, st))
        (o1, s1), (o0, s0) = res
        assert torch.isfinite(o1.float()).all() and torch.isfinite(s1).all(), f"{dt}: the NaN buffer was read"
        assert torch.equal(o1, o0) and torch.equal(s1, s0), f"{dt}: result depends on the unused buffer"
        ro, rs = _oracle_cte(d, False)
        tol = TOL_F32 if dt == "f32" else TOL_BF16
        assert_close(host(o1), ro, tol, 2, f"{dt} out")
        assert_close(host(s1), rs, tol, 2, f"{dt} state")


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------
def _tkg_args(d):
    return [d[n] for n in ("q", "k", "v", "b", "a", "A_log", "dt_bias", "z", "norm_weight", "state_in")]


def _oracle_tkg(d, rms_eps=1e-6):
    y, s = c_ref.tkg_unrounded(*[x.f64() for x in _tkg_args(d)], d["num_v_heads"], rms_eps=rms_eps)
    return gdn_ref.bf16_round(y), s


TKG_CASES = [
    # (B, Hv, K, V, dtype)
    (3, 4, 64, 32, "bf16"),
    (2, 5, 128, 128, "f32"),
    (1, 2, 40, 72, "bf16"),
    (4, 1, 8, 8, "bf16"),
]


@pytest.mark.parametrize("case", TKG_CASES, ids=lambda c: "B{}_Hv{}_K{}_V{}_{}".format(*c))
def test_tkg_matches_oracle(gpu_lib, case):
    B, Hv, K, V, dt = case
    d = inputs.tkg_inputs(B, Hv, K, V, dtype=dt, seed=2000 + K + V)
    y, s = gpu_lib.gdn_tkg(*[dev(x) for x in _tkg_args(d)])
    _sync()
    ry, rs = _oracle_tkg(d)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(host(s), rs, tol, 1, "state")
    assert_close(host(y), ry, TOL_BF16, 1, "out")


def test_tkg_bh1024_workload_in_place(gpu_lib):
    """B=32, Hv=32 (BH=1024), K=V=128, bf16 q/k/v/z: out-of-place and in-place."""
    import torch
    d = inputs.workload_inputs("tkg_b32_hv32_d128")
    args = [dev(x) for x in _tkg_args(d)]
    y, s = gpu_lib.gdn_tkg(*args)
    _sync()
    ry, rs = _oracle_tkg(d)
    assert_close(host(s), rs, TOL_BF16, 1, "state")
    assert_close(host(y), ry, TOL_BF16, 1, "out")
    st = args[-1].clone()
    y2, s2 = gpu_lib.gdn_tkg(*args[:-1], st, state_out=st)
    _sync()
    assert s2.data_ptr() == st.data_ptr()
    assert torch.equal(s2, s) and torch.equal(y2, y)


@pytest.mark.parametrize("B,Hv,dt", [(75, 20, "bf16"), (70, 30, "f32"), (33, 31, "bf16")],
                         ids=["BH1500_bf16", "BH2100_f32", "BH1023_bf16"])
def test_tkg_heads_over_several_launches(gpu_lib, B, Hv, dt):
    """More heads than one round (1024) go out as several launches of an even
    share each (1500 -> 2 x 750, 2100 -> 3 x 700; 1023 stays one launch): every
    head, out-of-place and in-place, against the oracle."""
    import torch
    d = inputs.tkg_inputs(B, Hv, 128, 128, dtype=dt, seed=2200 + B * Hv)
    args = [dev(x) for x in _tkg_args(d)]
    y, s = gpu_lib.gdn_tkg(*args)
    _sync()
    ry, rs = _oracle_tkg(d)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert_close(host(s), rs, tol, 1, "state")
    assert_close(host(y), ry, TOL_BF16, 1, "out")
    st = args[-1].clone()
    y2, s2 = gpu_lib.gdn_tkg(*args[:-1], st, state_out=st)
    _sync()
    assert torch.equal(s2, s) and torch.equal(y2, y)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-5])
def test_tkg_rms_eps_sweep(gpu_lib, eps):
    d = inputs.tkg_inputs(2, 8, 128, 128, seed=2100)
    y, _ = gpu_lib.gdn_tkg(*[dev(x) for x in _tkg_args(d)], rms_eps=eps)
    _sync()
    ry, _ = _oracle_tkg(d, rms_eps=eps)
    assert_close(host(y), ry, TOL_BF16, 1, f"out eps={eps}")


def test_decode_after_prefill(gpu_lib):
    """Prefill S tokens, then one decode step from the returned state, equals the
    oracle run the same way (state hand-off between the two entry points)."""
    import torch
    B, Hk, Hv, S, D = 1, 2, 4, 192, 128
    d = inputs.cte_inputs(B, Hk, Hv, S, D, D, dtype="bf16", state_std=0.05, seed=2200)
    _, st = gpu_lib.gdn_cte(dev(d["query"]), dev(d["key"]), dev(d["value"]), dev(d["g_log"]),
                            dev(d["beta"]), d["scale"], recurrent_state=dev(d["recurrent_state"]).clone())
    t = inputs.tkg_inputs(B, Hv, D, D, seed=2201)
    y, s1 = gpu_lib.gdn_tkg(*[dev(x) for x in _tkg_args(t)[:-1]], st.reshape(B * Hv, D, D).contiguous())
    _sync()
    _, rs = c_ref.cte(d["query"].f64(), d["key"].f64(), d["value"].f64(), d["g_log"].f64(),
                      d["beta"].f64(), d["scale"], d["recurrent_state"].f64())
    args = [x.f64() for x in _tkg_args(t)[:-1]] + [rs.reshape(B * Hv, D, D)]
    ry, rs1 = c_ref.tkg_unrounded(*args, Hv)
    assert_close(host(s1), rs1, TOL_BF16, 1, "state")
    assert_close(host(y), gdn_ref.bf16_round(ry), TOL_BF16, 1, "out")


# ---------------------------------------------------------------------------
# fused decode layer
# ---------------------------------------------------------------------------
BLOCK_KEYS = ("hidden", "W_in_qkv", "W_in_z", "W_in_a", "W_in_b", "conv_weight", "conv_state",
              "A_log", "dt_bias", "norm_weight", "recurrent_state")


def _oracle_block(d):
    a = [d[n].f64() for n in BLOCK_KEYS]
    return gdn_ref.block_tkg(*a, d["num_k_heads"], d["num_v_heads"], d["head_k_dim"], d["head_v_dim"])


def _check_block(gpu_out, d):
    y, cs, rs = (host(t) for t in gpu_out)
    ry, rcs, rrs = _oracle_block(d)
    B = y.shape[0]
    Hv, Dv = d["num_v_heads"], d["head_v_dim"]
    assert_close(rs, rrs, TOL_BF16, 2, "recurrent_state")
    assert_close(y.reshape(B * Hv, Dv), ry.reshape(B * Hv, Dv), TOL_BF16, 1, "out")
    # the slid part of the window is copied bit for bit; the new column is the
    # bf16-rounded projection, held to the fp32 rounding interval of its sum
    np.testing.assert_array_equal(cs[:, :, :-1], rcs[:, :, :-1])
    assert_bf16_sums_match(cs[:, :, -1:], rcs[:, :, -1:], d["hidden"].f64(), d["W_in_qkv"].f64(),
                           "conv_state new column")


# H = 1024 / 4096 take the fully unrolled K loops; B = 70 spans two batch tiles
# with a ragged second one; Hv = 8 takes the vector a|b tile; windows of 6 and
# 8 take the generic conv epilogue up to the longest window the API accepts;
# B*Hv = 1120 and 1040 run the decode step as two launches (of 560 and 520
# heads), the first at the model's head dims
@pytest.mark.parametrize("case", [(3, 256, 2, 4, 32, 32, 4), (5, 384, 1, 2, 64, 48, 3), (2, 128, 2, 2, 16, 16, 1),
                                  (70, 1024, 2, 8, 32, 32, 4), (17, 4096, 1, 8, 16, 24, 2),
                                  (4, 256, 2, 4, 32, 32, 8), (3, 128, 1, 2, 16, 24, 6),
                                  (35, 2048, 16, 32, 128, 128, 4), (130, 256, 2, 8, 32, 32, 4)],
                         ids=lambda c: "B{}_H{}_Hk{}_Hv{}_Dk{}_Dv{}_W{}".format(*c))
def test_block_small(gpu_lib, case):
    B, H, Hk, Hv, Dk, Dv, W = case
    d = inputs.block_inputs(B, H, Hk, Hv, Dk, Dv, K_win=W, w_std=0.05, seed=3000 + H)
    out = gpu_lib.gdn_block_tkg(*[dev(d[n]) for n in BLOCK_KEYS])
    _sync()
    _check_block(out, d)


def test_block_b64_workload_in_place(gpu_lib):
    """B=64, H=2048, Hk=16, Hv=32, D=128, K_win=4: functional call against the
    oracle, then the in-place call (caches aliased) gives the same bits."""
    import torch
    d = inputs.workload_inputs("block_b64_h2048_hk16_hv32_d128")
    args = [dev(d[n]) for n in BLOCK_KEYS]
    out = gpu_lib.gdn_block_tkg(*args)
    _sync()
    _check_block(out, d)
    cs, rs = args[6].clone(), args[10].clone()
    out2 = gpu_lib.gdn_block_tkg(*args[:6], cs, *args[7:10], rs, conv_state_out=cs, recurrent_state_out=rs)
    _sync()
    for a, b in zip(out, out2):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# the fused prefill and the prefill layer at the shapes bench.py times
# ---------------------------------------------------------------------------
def test_cte_fused_bench_shape_all_heads(gpu_lib):
    """gdn_cte_fused at B=1, Hk=16, Hv=32, S=4096, D=128, bf16, supplied state
    (the bench's fused-prefill call and seed): every value head's output and
    state against the oracle."""
    B, Hk, Hv, S, D = 1, 16, 32, 4096, 128
    d = inputs.cte_fused_inputs(B, Hk, Hv, S, D, D, dtype="bf16", state_std=0.05, seed=11)
    st = dev(d["recurrent_state"]).clone()
    y, state = gpu_lib.gdn_cte_fused(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["b"]), dev(d["a"]),
                                     dev(d["A_log"]), dev(d["dt_bias"]), dev(d["z"]), dev(d["norm_weight"]),
                                     recurrent_state=st)
    _sync()
    ry, rs = _oracle_cte_fused(d, d["recurrent_state"].f64())
    assert_close(host(y), ry, TOL_BF16, 2, "out")
    assert_close(host(state), rs, TOL_BF16, 2, "state")


def _oracle_cte_fused(d, s0):
    """oracle.gdn_ref.cte_fused with its recurrence on the C twin (the same
    token-by-token definition, OpenMP over heads), for the bench shapes."""
    Dk = d["q"].shape[-1]
    q_unit, k_unit = gdn_ref.l2norm(d["q"].f64()), gdn_ref.l2norm(d["k"].f64())
    beta = gdn_ref.sigmoid(d["b"].f64())
    rate = np.exp(d["A_log"].f64())[None, :, None]
    g = -rate * gdn_ref.softplus(d["a"].f64() + d["dt_bias"].f64()[None, :, None])
    O, S1 = c_ref.cte(q_unit, k_unit, d["v"].f64(), g, beta, 1.0 / math.sqrt(Dk), s0)
    return gdn_ref.rms_norm_gated(O, d["z"].f64(), d["norm_weight"].f64()), S1


def test_block_cte_bench_shape_all_heads(gpu_lib):
    """gdn_block_cte at B=1, S=4096, H=2048, Hk=16, Hv=32, D=128, K_win=4 with the
    caches updated in place (the bench's prefill-layer call and seed): every
    value head of the output and the recurrent state against the oracle's
    layer, and the final conv window against the oracle's last K_win
    projections."""
    B, S, H, Hk, Hv, D, Kw = 1, 4096, 2048, 16, 32, 128, 4
    d = inputs.block_cte_inputs(B, S, H, Hk, Hv, D, D, K_win=Kw, seed=12)
    cs = dev(d["conv_state"]).clone()
    rs = dev(d["recurrent_state"]).clone()
    args = [dev(d[n]) for n in ("hidden", "W_in_qkv", "W_in_z", "W_in_a", "W_in_b", "conv_weight")]
    out, cs1, rs1 = gpu_lib.gdn_block_cte(*args, cs, dev(d["A_log"]), dev(d["dt_bias"]), dev(d["norm_weight"]), rs,
                                          conv_state_out=cs, recurrent_state_out=rs)
    _sync()
    out, cs1, rs1 = host(out), host(cs1), host(rs1)
    f = {n: d[n].f64() for n in ("hidden", "W_in_qkv", "W_in_z", "W_in_a", "W_in_b", "conv_weight", "conv_state",
                                 "A_log", "dt_bias", "norm_weight", "recurrent_state")}
    # the oracle layer (gdn_ref.block_cte) with its recurrence on the C twin
    key_dim = Hk * D
    x = f["hidden"].reshape(B * S, H)
    mixed = gdn_ref.in_proj(x, f["W_in_qkv"]).reshape(B, S, -1)
    zz = gdn_ref.in_proj(x, f["W_in_z"]).reshape(B, S, Hv, D).transpose(0, 2, 1, 3)
    aa = gdn_ref.in_proj(x, f["W_in_a"]).reshape(B, S, Hv).transpose(0, 2, 1)
    bb = gdn_ref.in_proj(x, f["W_in_b"]).reshape(B, S, Hv).transpose(0, 2, 1)
    conv_out, window = gdn_ref.conv1d_prefill(mixed, f["conv_state"], f["conv_weight"])
    conv_out = gdn_ref.bf16_round(conv_out)
    q = conv_out[:, :, :key_dim].reshape(B, S, Hk, D).transpose(0, 2, 1, 3)
    k = conv_out[:, :, key_dim:2 * key_dim].reshape(B, S, Hk, D).transpose(0, 2, 1, 3)
    v = conv_out[:, :, 2 * key_dim:].reshape(B, S, Hv, D).transpose(0, 2, 1, 3)
    sub = {n: _F64(a) for n, a in (("q", q), ("k", k), ("v", v), ("b", bb), ("a", aa), ("A_log", f["A_log"]),
                                   ("dt_bias", f["dt_bias"]), ("z", zz), ("norm_weight", f["norm_weight"]))}
    ry, rrs = _oracle_cte_fused(sub, f["recurrent_state"])
    ry = ry.transpose(0, 2, 1, 3).reshape(B, S, Hv * D)
    assert_close(out.reshape(B * S, Hv, D).transpose(1, 0, 2), ry.reshape(B * S, Hv, D).transpose(1, 0, 2),
                 TOL_BF16, 1, "out (per value head)")
    assert_close(rs1, rrs, TOL_BF16, 2, "recurrent state")
    assert_bf16_sums_match(cs1, window, f["hidden"][:, -Kw:], f["W_in_qkv"], "conv window")


class _F64:
    """A float64 array in the place of an inputs.Arr (its .f64() and .shape)."""
    def __init__(self, a):
        self.a = np.asarray(a, np.float64)
        self.shape = self.a.shape

    def f64(self):
        return self.a


def assert_bf16_sums_match(x, ref, hidden, W, what, max_frac=1e-2):
    """x (GPU) and ref (oracle) are bf16 roundings of the dot products hidden @ W
    over K terms, x accumulated in fp32, ref rounded from the exact fp64 sum.
    Any fp32 summation order is within K 2^-24 sum|terms| of the exact sum, so
    every x must be the bf16 rounding of some value in that interval; and the
    two may differ only where a sum sits that close to a rounding midpoint,
    which is rare."""
    K = hidden.shape[-1]
    exact = np.matmul(hidden, W).transpose(0, 2, 1)
    bound = K * 2.0 ** -24 * np.matmul(np.abs(hidden), np.abs(W)).transpose(0, 2, 1)
    lo, hi = gdn_ref.bf16_round(exact - bound), gdn_ref.bf16_round(exact + bound)
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    bad = (x < lo) | (x > hi)
    assert not bad.any(), (f"{what}: {int(bad.sum())} values outside the fp32 rounding interval; at "
                           f"{np.argwhere(bad)[:8].tolist()}: gpu {x[bad][:8]}, ref {ref[bad][:8]}")
    frac = float((x != ref).mean())
    assert frac <= max_frac, f"{what}: {frac:.2%} of the values differ from the oracle's rounding"


# ---------------------------------------------------------------------------
# graph capture of the other entry points (the library records no memset)
# ---------------------------------------------------------------------------
def _check_graph_replays(call, fresh, outputs, what):
    """call() launches on the current stream and writes `outputs`; fresh()
    restores every buffer the call updates in place.  Capture once, then replay
    three times with eager work and syncs in between: each replay must equal
    the eager call bit for bit."""
    import torch
    fresh()
    call()
    _sync()
    refs = [o.clone() for o in outputs]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fresh()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            call()
    for _ in range(3):
        for o in outputs:
            o.zero_()
        fresh()
        _sync()
        graph.replay()
        _sync()
        for o, r in zip(outputs, refs):
            assert torch.equal(o, r), f"{what}: a graph replay differs from the eager call"


def test_tkg_and_block_tkg_inside_graph_capture(gpu_lib):
    """The decode step and the decode layer with their caches updated in place,
    as a serving loop captures them."""
    import torch
    t = inputs.tkg_inputs(4, 8, 128, 128, seed=71)
    names = ("q", "k", "v", "b", "a", "A_log", "dt_bias", "z", "norm_weight", "state_in")
    a = [dev(t[n]) for n in names]
    s0, st = a[9].clone(), a[9]
    y = torch.empty((32, 128), dtype=torch.bfloat16, device=st.device)

    def fresh():
        st.copy_(s0)
    _check_graph_replays(lambda: gpu_lib.gdn_tkg(*a[:9], st, state_out=st, out=y), fresh, [y, st], "gdn_tkg")

    b = inputs.block_inputs(8, 512, 2, 4, 64, 64, seed=72)
    args = [dev(b[n]) for n in BLOCK_KEYS]
    cs0, rs0 = args[6].clone(), args[10].clone()
    cs, rs = args[6], args[10]
    out = torch.empty((8, 1, 4 * 64), dtype=torch.bfloat16, device=cs.device)

    def fresh_b():
        cs.copy_(cs0)
        rs.copy_(rs0)
    _check_graph_replays(lambda: gpu_lib.gdn_block_tkg(*args, conv_state_out=cs, recurrent_state_out=rs, out=out),
                         fresh_b, [out, cs, rs], "gdn_block_tkg")


def test_fused_prefill_and_prefill_layer_inside_graph_capture(gpu_lib):
    """gdn_cte_fused (the folded prologue) and gdn_block_cte (GEMM, conv, fused
    prefill, output norm; caches in place) captured and replayed."""
    import torch
    d = inputs.cte_fused_inputs(1, 2, 4, 300, 128, 128, dtype="bf16", state_std=0.05, seed=73)
    keys = ("q", "k", "v", "b", "a", "A_log", "dt_bias", "z", "norm_weight")
    a = [dev(d[n]) for n in keys]
    s0 = dev(d["recurrent_state"])
    st = s0.clone()
    y = torch.empty((1, 4, 300, 128), dtype=torch.bfloat16, device=st.device)

    def fresh():
        st.copy_(s0)
    _check_graph_replays(lambda: gpu_lib.gdn_cte_fused(*a, recurrent_state=st, out=y), fresh, [y, st],
                         "gdn_cte_fused")

    c = inputs.block_cte_inputs(1, 200, 256, 2, 4, 64, 64, K_win=4, seed=74)
    args = [dev(c[n]) for n in ("hidden", "W_in_qkv", "W_in_z", "W_in_a", "W_in_b", "conv_weight")]
    cs0, rs0 = dev(c["conv_state"]), dev(c["recurrent_state"])
    cs, rs = cs0.clone(), rs0.clone()
    rest = [dev(c[n]) for n in ("A_log", "dt_bias", "norm_weight")]
    out = torch.empty((1, 200, 4 * 64), dtype=torch.bfloat16, device=cs.device)

    def fresh_c():
        cs.copy_(cs0)
        rs.copy_(rs0)
    _check_graph_replays(lambda: gpu_lib.gdn_block_cte(*args, cs, *rest, rs, conv_state_out=cs,
                                                       recurrent_state_out=rs, out=out),
                         fresh_c, [out, cs, rs], "gdn_block_cte")
