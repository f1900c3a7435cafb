"""gdn_cte_noalloc (the prefill on the library's fixed scratch) through the C
ABI against gdn_cte with a caller-owned workspace: the same bits, and the
oracle's bar, on two calls in a row (the second smaller, so it runs on what
the first left in the scratch); a call that needs more scratch than the
library holds is refused without touching its outputs."""
import ctypes

import numpy as np
import pytest

from gated_delta_rule_cte_amd import inputs
from oracle import c_ref
from tests.gpu_util import TOL_BF16, TOL_F32, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(gdn, lib, q, k, v, g, be, scale, st, has_init, out, dtype):
    import torch
    B, Hk, S, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[3]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.gdn_cte_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(be), scale, _ptr(st), has_init, _ptr(out),
                               B, Hk, Hv, S, Dk, Dv, dtype, 0, stream)


@pytest.mark.parametrize("cases", [
    # (B, Hk, Hv, S, Dk, Dv, dtype, with_state), the second call smaller
    ((1, 2, 4, 1500, 128, 128, "bf16", True), (1, 1, 2, 333, 64, 64, "bf16", False)),
    ((1, 2, 2, 200, 64, 64, "f32", True), (1, 1, 1, 77, 32, 48, "f32", True)),
], ids=["bf16", "f32"])
def test_noalloc_matches_gdn_cte_on_consecutive_calls(gpu_lib, cases):
    import torch
    lib = gpu_lib.load()
    for i, (B, Hk, Hv, S, Dk, Dv, dt, ws) in enumerate(cases):
        print(f"noalloc call {i}: B={B} Hk={Hk} Hv={Hv} S={S} Dk={Dk} Dv={Dv} {dt} state={ws}", flush=True)
        d = inputs.cte_inputs(B, Hk, Hv, S, Dk, Dv, dtype=dt, state_std=0.05 if ws else None, seed=4000 + i)
        q, k, v, g, be = (dev(d[n]) for n in ("query", "key", "value", "g_log", "beta"))
        code = gpu_lib.GDN_BF16 if dt == "bf16" else gpu_lib.GDN_F32
        s0 = dev(d["recurrent_state"]) if ws else torch.zeros((B, Hv, Dk, Dv), dtype=torch.float32, device=q.device)
        st = s0.clone()
        out = torch.empty_like(v)
        rc = _noalloc(gpu_lib, lib, q, k, v, g, be, d["scale"], st, int(ws), out, code)
        assert rc == 0, lib.gdn_last_error().decode()
        ref_out, ref_st = gpu_lib.gdn_cte(q, k, v, g, be, d["scale"], recurrent_state=s0.clone() if ws else None)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"call {i}: output differs from gdn_cte"
        assert torch.equal(st, ref_st), f"call {i}: state differs from gdn_cte"
        ro, rs = c_ref.cte(d["query"].f64(), d["key"].f64(), d["value"].f64(), d["g_log"].f64(), d["beta"].f64(),
                           d["scale"], d["recurrent_state"].f64() if ws else None)
        tol = TOL_F32 if dt == "f32" else TOL_BF16
        assert_close(host(out), ro, tol, 2, f"call {i} out")
        assert_close(host(st), rs, tol, 2, f"call {i} state")


def test_noalloc_refuses_calls_beyond_its_scratch(gpu_lib):
    """A shape whose workspace exceeds the fixed scratch: GDN_ERR_WORKSPACE with
    a message, and the output and state buffers keep their contents."""
    import torch
    lib = gpu_lib.load()
    B, Hk, Hv, Dk, Dv = 1, 1, 64, 64, 64
    S = 64
    while lib.gdn_cte_workspace_size(B, Hk, Hv, S, Dk, Dv, gpu_lib.GDN_BF16) <= (64 << 20):
        S *= 2
    print(f"oversized call: B={B} Hv={Hv} S={S}", flush=True)
    bf = torch.bfloat16
    q = torch.zeros((B, Hk, S, Dk), dtype=bf, device="cuda")
    v = torch.zeros((B, Hv, S, Dv), dtype=bf, device="cuda")
    g = torch.zeros((B, Hv, S), dtype=torch.float32, device="cuda")
    st = torch.full((B, Hv, Dk, Dv), 7.0, device="cuda")
    out = torch.full_like(v, 3.0)
    rc = _noalloc(gpu_lib, lib, q, q, v, g, g, 0.125, st, 1, out, gpu_lib.GDN_BF16)
    torch.cuda.synchronize()
    assert rc == -6, f"status {rc}"
    assert "scratch" in lib.gdn_last_error().decode()
    assert torch.all(st == 7.0) and torch.all(out == 3.0)
