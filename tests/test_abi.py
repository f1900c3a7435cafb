"""C-ABI contract tests that need no GPU: libgdn loads, exports every symbol
include/gdn.h declares, and rejects bad arguments with the documented status
before any HIP call (fake, never-dereferenced device addresses are passed)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_cte_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

A = 0x10000000      # fake 16-byte aligned addresses, far apart
STEP = 0x10000000


def _gpu_visible():
    """True when a HIP device may be visible to this process.  Checked without
    initialising HIP: the KFD device node, or torch's device count."""
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# A call whose arguments all pass validation reaches the device check and,
# on a machine with a gfx950, launches kernels.  With the fake addresses used
# here that would fault the GPU, so such calls run only where no GPU is
# visible (where the device check, the last one, reports GDN_ERR_DEVICE).
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="valid arguments with fake device addresses would "
                                 "launch kernels on the visible GPU")


def addrs(n):
    return [ctypes.c_void_p(A + i * STEP) for i in range(n)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built (run python -m gated_delta_rule_cte_amd.build)")
    return gdn.load()


def test_header_declarations_match_exports(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^(?:int|size_t|const char\*)\s+(gdn_\w+)\(", text, re.M))
    assert declared == set(gdn.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.gdn_version() == 100
    for code, name in gdn.STATUS.items():
        assert lib.gdn_status_string(code).decode() == name
    assert lib.gdn_status_string(-99).decode() == "GDN_ERR_UNKNOWN"


def cte_call(lib, **kw):
    args = dict(B=1, Hk=2, Hv=4, S=128, Dk=64, Dv=64, dtype=gdn.GDN_BF16, algorithm=0,
                has_init=1)
    args.update(kw)
    p = addrs(7)
    ptrs = kw.get("ptrs", p)
    need = lib.gdn_cte_workspace_size(args["B"], args["Hk"], args["Hv"], args["S"], args["Dk"], args["Dv"],
                                      args["dtype"])
    ws = kw.get("ws", ctypes.c_void_p(A + 20 * STEP))
    return lib.gdn_cte(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], 0.125, ptrs[5], args["has_init"],
                       ptrs[6], args["B"], args["Hk"], args["Hv"], args["S"], args["Dk"], args["Dv"],
                       args["dtype"], args["algorithm"], ws, kw.get("ws_bytes", need), None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), -3),
    (dict(algorithm=2), -7),
    (dict(algorithm=-1), -7),
    (dict(Hv=3), -2),
    (dict(Hk=0), -2),
    (dict(Dk=130), -2),
    (dict(Dv=12), -2),
    (dict(Dk=0), -2),
    (dict(S=-1), -2),
    (dict(B=-2), -2),
])
def test_cte_rejects_bad_shapes(lib, kw, status):
    assert cte_call(lib, **kw) == status
    assert lib.gdn_last_error().decode() != ""


def test_cte_rejects_null_misaligned_and_aliased(lib):
    p = addrs(7)
    bad = list(p)
    bad[2] = None
    assert cte_call(lib, ptrs=bad) == -1
    bad = list(p)
    bad[0] = ctypes.c_void_p(A + 8)
    assert cte_call(lib, ptrs=bad) == -4
    bad = list(p)
    bad[6] = ctypes.c_void_p(p[2].value + 64)       # out inside value
    assert cte_call(lib, ptrs=bad) == -5
    bad = list(p)
    bad[5] = ctypes.c_void_p(p[3].value)            # state on top of g_log
    assert cte_call(lib, ptrs=bad) == -5


def test_cte_workspace_checks(lib):
    need = lib.gdn_cte_workspace_size(1, 2, 4, 128, 64, 64, gdn.GDN_BF16)
    assert need == 4 * 2 * 2 * 64 * 64 * 2          # Hv * chunks * (T, P) * 64 * 64 * bf16
    assert lib.gdn_cte_workspace_size(1, 2, 4, 0, 64, 64, gdn.GDN_BF16) == 0
    assert lib.gdn_cte_workspace_size(1, 2, 4, 65, 64, 64, gdn.GDN_F32) == 4 * 2 * 2 * 64 * 64 * 4
    assert cte_call(lib, ws=None) == -6
    assert cte_call(lib, ws_bytes=need - 1) == -6
    assert cte_call(lib, ws=ctypes.c_void_p(A + 20 * STEP + 16)) == -4
    assert cte_call(lib, ws=ctypes.c_void_p(A + 2 * STEP)) == -5   # on top of value




def test_cte_empty_batch_is_a_no_op(lib):
    assert cte_call(lib, B=0) == 0
    assert lib.gdn_last_error().decode() == ""


def tkg_call(lib, ptrs=None, BH=64, Hv=32, K=128, V=128, dtype=gdn.GDN_BF16, eps=1e-6):
    p = ptrs or addrs(12)
    return lib.gdn_tkg(*p, BH, Hv, K, V, dtype, eps, None)


def test_tkg_checks(lib):
    assert tkg_call(lib, Hv=5) == -2
    assert tkg_call(lib, K=136) == -2
    assert tkg_call(lib, V=4) == -2
    assert tkg_call(lib, dtype=3) == -3
    assert tkg_call(lib, eps=-1.0) == -2
    assert tkg_call(lib, BH=0) == 0
    p = addrs(12)
    q = list(p)
    q[10] = ctypes.c_void_p(p[9].value + 4096)       # partial overlap: rejected
    assert tkg_call(lib, ptrs=q) == -5
    q = list(p)
    q[11] = ctypes.c_void_p(p[3].value)              # out on top of v
    assert tkg_call(lib, ptrs=q) == -5
    q = list(p)
    q[0] = None
    assert tkg_call(lib, ptrs=q) == -1


def block_call(lib, ptrs=None, ws=None, ws_bytes=None, **kw):
    d = dict(B=64, H=2048, Hk=16, Hv=32, Dk=128, Dv=128, K_win=4)
    d.update(kw)
    need = lib.gdn_block_tkg_workspace_size(d["B"], d["H"], d["Hk"], d["Hv"], d["Dk"], d["Dv"], d["K_win"])
    p = ptrs or addrs(14)
    ws = ctypes.c_void_p(A + 20 * STEP) if ws is None else ws
    return lib.gdn_block_tkg(*p, d["B"], d["H"], d["Hk"], d["Hv"], d["Dk"], d["Dv"], d["K_win"], 1e-6,
                             ws, need if ws_bytes is None else ws_bytes, None)


def test_block_checks(lib):
    need = lib.gdn_block_tkg_workspace_size(64, 2048, 16, 32, 128, 128, 4)
    conv_dim = 2 * 16 * 128 + 32 * 128
    assert need >= 64 * conv_dim * 2 + 64 * 4096 * 2 + 2 * 64 * 32 * 4
    assert block_call(lib, H=2000) == -2
    assert block_call(lib, Hv=24) == -2
    assert block_call(lib, K_win=9) == -2
    assert block_call(lib, ws_bytes=need - 1) == -6
    assert block_call(lib, ws=ctypes.c_void_p(0), ws_bytes=need) == -6
    assert block_call(lib, B=0) == 0
    p = addrs(14)
    q = list(p)
    q[11] = ctypes.c_void_p(p[0].value)              # out on top of hidden
    assert block_call(lib, ptrs=q) == -5


def test_binding_fails_loudly_without_library(tmp_path):
    saved = gdn._lib
    try:
        gdn._lib = None
        with pytest.raises(ImportError):
            gdn.load(str(tmp_path / "missing.so"))
    finally:
        gdn._lib = saved


def fused_call(lib, ptrs=None, B=1, Hk=2, Hv=4, S=100, Dk=64, Dv=64, dtype=gdn.GDN_BF16, algorithm=0,
               eps=1e-6, ws="auto", ws_bytes=None):
    p = ptrs or addrs(11)
    need = lib.gdn_cte_fused_workspace_size(B, Hk, Hv, S, Dk, Dv, dtype)
    w = ctypes.c_void_p(A + 20 * STEP) if ws == "auto" else ws
    return lib.gdn_cte_fused(*p[:10], 1, p[10], B, Hk, Hv, S, Dk, Dv, dtype, algorithm, eps, w,
                             need if ws_bytes is None else ws_bytes, None)


def test_cte_fused_checks(lib):
    """gdn_cte_fused: every argument check, before any HIP call."""
    assert fused_call(lib, dtype=9) == -3
    assert fused_call(lib, algorithm=2) == -7
    assert fused_call(lib, Hv=3) == -2
    assert fused_call(lib, Dk=130) == -2
    assert fused_call(lib, S=-1) == -2
    assert fused_call(lib, eps=-1.0) == -2
    bad = addrs(11)
    bad[2] = None                                   # v
    assert fused_call(lib, ptrs=bad) == -1
    bad = addrs(11)
    bad[7] = ctypes.c_void_p(bad[7].value + 4)      # z misaligned
    assert fused_call(lib, ptrs=bad) == -4
    bad = addrs(11)
    bad[10] = ctypes.c_void_p(bad[0].value + 64)    # out inside q
    assert fused_call(lib, ptrs=bad) == -5
    bad = addrs(11)
    bad[9] = ctypes.c_void_p(bad[3].value)          # state on top of b
    assert fused_call(lib, ptrs=bad) == -5
    need = lib.gdn_cte_fused_workspace_size(1, 2, 4, 100, 64, 64, gdn.GDN_BF16)
    assert need > lib.gdn_cte_workspace_size(1, 2, 4, 100, 64, 64, gdn.GDN_BF16)
    assert fused_call(lib, ws=None) == -6
    assert fused_call(lib, ws_bytes=need - 1) == -6
    assert fused_call(lib, ws=ctypes.c_void_p(A + 20 * STEP + 16)) == -4
    assert fused_call(lib, ws=ctypes.c_void_p(A + 2 * STEP)) == -5     # on top of v
    assert fused_call(lib, B=0) == 0


def block_cte_call(lib, ptrs=None, B=2, S=16, H=128, Hk=2, Hv=4, Dk=32, Dv=32, K_win=4, algorithm=0,
                   eps=1e-6, ws="auto", ws_bytes=None):
    p = ptrs or addrs(14)
    need = lib.gdn_block_cte_workspace_size(B, S, H, Hk, Hv, Dk, Dv, K_win)
    w = ctypes.c_void_p(A + 30 * STEP) if ws == "auto" else ws
    return lib.gdn_block_cte(*p, B, S, H, Hk, Hv, Dk, Dv, K_win, algorithm, eps, w,
                             need if ws_bytes is None else ws_bytes, None)


def test_block_cte_checks(lib):
    """gdn_block_cte: every argument check, before any HIP call; the caches may
    alias their inputs exactly but not partly."""
    assert block_cte_call(lib, H=100) == -2
    assert block_cte_call(lib, K_win=9) == -2
    assert block_cte_call(lib, Hv=3) == -2
    assert block_cte_call(lib, Dv=12) == -2
    assert block_cte_call(lib, algorithm=5) == -7
    bad = addrs(14)
    bad[1] = None                                   # W_in_qkv
    assert block_cte_call(lib, ptrs=bad) == -1
    bad = addrs(14)
    bad[11] = ctypes.c_void_p(bad[0].value + 32)    # out inside hidden
    assert block_cte_call(lib, ptrs=bad) == -5
    bad = addrs(14)
    bad[12] = ctypes.c_void_p(bad[6].value + 16)    # conv_state_out partly over conv_state_in
    assert block_cte_call(lib, ptrs=bad) == -5
    assert block_cte_call(lib, ws=None) == -6
    need = lib.gdn_block_cte_workspace_size(2, 16, 128, 2, 4, 32, 32, 4)
    assert block_cte_call(lib, ws_bytes=need - 1) == -6
    assert block_cte_call(lib, ws=ctypes.c_void_p(A + 30 * STEP + 128)) == -4
    assert block_cte_call(lib, B=0) == 0


@no_gpu_only
def test_valid_calls_reach_the_device_check(lib):
    """Every argument check passes (including exact in/out aliases and a
    sequence with no chunks); the device check, which is last, reports that
    there is no gfx950."""
    assert cte_call(lib) == -9
    assert "device" in lib.gdn_last_error().decode().lower()
    assert cte_call(lib, S=0, ws=None) == -9                        # no workspace needed
    p = addrs(12)
    q = list(p)
    q[10] = p[9]                                                    # state_out == state_in
    assert tkg_call(lib, ptrs=q) == -9
    assert tkg_call(lib) == -9
    assert block_call(lib, Dk=120) == -9                            # 120 is a multiple of 8
    p = addrs(14)
    q = list(p)
    q[12] = p[6]                                                    # conv_state_out == conv_state_in
    q[13] = p[10]                                                   # recurrent_state_out == in
    assert block_call(lib, ptrs=q) == -9
    assert block_call(lib) == -9
    assert fused_call(lib) == -9
    inplace = addrs(14)
    inplace[12], inplace[13] = inplace[6], inplace[10]
    assert block_cte_call(lib, ptrs=inplace) == -9                  # exact aliases are valid
    assert block_cte_call(lib) == -9


def _block_cpu_args(B=2, S=None, H=128, Hk=1, Hv=2, D=16, K_win=4):
    """Correctly shaped CPU tensors for the decode layer (S=None) or the prefill
    layer; the binding checks every shape before it looks at the device."""
    import torch
    bf, f = torch.bfloat16, torch.float32
    conv_dim = 2 * Hk * D + Hv * D
    hid = (B, 1, H) if S is None else (B, S, H)
    return [torch.zeros(hid, dtype=bf), torch.zeros((H, conv_dim), dtype=bf), torch.zeros((H, Hv * D), dtype=bf),
            torch.zeros((H, Hv), dtype=bf), torch.zeros((H, Hv), dtype=bf), torch.zeros((conv_dim, K_win), dtype=f),
            torch.zeros((B, conv_dim, K_win), dtype=bf), torch.zeros(Hv, dtype=f), torch.zeros(Hv, dtype=f),
            torch.zeros(D, dtype=f), torch.zeros((B, Hv, D, D), dtype=f)]


@pytest.mark.parametrize("layer", ["decode", "prefill"])
def test_binding_checks_caller_outputs_before_any_launch(lib, layer):
    """A caller-supplied output (or workspace) of the wrong shape, dtype or
    layout raises in the binding before the library is called; with every
    shape right, the next check is the device (these are CPU tensors)."""
    import torch
    S = None if layer == "decode" else 3
    fn = gdn.gdn_block_tkg if layer == "decode" else gdn.gdn_block_cte
    a = _block_cpu_args(S=S)
    B, conv_dim, K_win = a[6].shape
    Hv, D = a[10].shape[1], a[10].shape[2]
    bad = {
        "conv_state_out": torch.zeros((B, conv_dim, K_win - 1), dtype=torch.bfloat16),
        "recurrent_state_out": torch.zeros((B, Hv, D, D), dtype=torch.bfloat16),
        "out": torch.zeros((B, 1 if S is None else S, Hv * D + 8), dtype=torch.bfloat16),
    }
    for name, t in bad.items():
        with pytest.raises((ValueError, TypeError), match=name):
            fn(*a, **{name: t})
    strided = torch.zeros((B, Hv, D, 2 * D), dtype=torch.float32)[..., :D]
    with pytest.raises(ValueError, match="recurrent_state_out must be contiguous"):
        fn(*a, recurrent_state_out=strided)
    if layer == "decode":
        with pytest.raises(TypeError, match="workspace"):
            fn(*a, workspace=torch.zeros(16, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU device"):
        fn(*a)


def test_binding_checks_prefill_and_decode_outputs(lib):
    import torch
    B, Hk, Hv, S, D = 1, 1, 2, 8, 16
    bf, f = torch.bfloat16, torch.float32
    q = torch.zeros((B, Hk, S, D), dtype=bf)
    v = torch.zeros((B, Hv, S, D), dtype=bf)
    g = torch.zeros((B, Hv, S), dtype=f)
    with pytest.raises(ValueError, match="out must have shape"):
        gdn.gdn_cte(q, q, v, g, g, out=torch.zeros((B, Hv, S, D + 8), dtype=bf))
    with pytest.raises(ValueError, match="recurrent_state must have shape"):
        gdn.gdn_cte(q, q, v, g, g, recurrent_state=torch.zeros((B, Hv, D, D + 8), dtype=f))
    with pytest.raises(ValueError, match="GPU device"):
        gdn.gdn_cte(q, q, v, g, g)
    BH = B * Hv
    x = torch.zeros((BH, D), dtype=bf)
    s = torch.zeros((BH, D, D), dtype=f)
    args = [x, x, x, torch.zeros(BH, dtype=f), torch.zeros(BH, dtype=f), torch.zeros(Hv, dtype=f),
            torch.zeros(Hv, dtype=f), x, torch.zeros(D, dtype=f), s]
    with pytest.raises(ValueError, match="state_out must have shape"):
        gdn.gdn_tkg(*args, state_out=torch.zeros((BH, D, D + 8), dtype=f))
    with pytest.raises(TypeError, match="out must be"):
        gdn.gdn_tkg(*args, out=torch.zeros((BH, D), dtype=f))
