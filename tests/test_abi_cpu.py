"""C-ABI checks that need no GPU: the library loads, exports exactly the
moe_* entry points include/moe.h declares, links no torch, and the host-side
argument checks return the documented status codes before any launch."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "grouped_gemm_router_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_exports_match_header():
    from grouped_gemm_router_amd import binding
    declared = _declared()
    assert len(declared) >= 11
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("moe_"))
    assert exported == declared
    assert sorted(binding.EXPORTS) == declared
    # nothing but the moe_ prefix (and toolchain-internal underscore symbols) is exported
    others = [l.split()[-1] for l in out.splitlines() if " T " in l and not l.split()[-1].startswith(("moe_", "_"))]
    assert others == []


def test_no_torch_dependency():
    out = subprocess.run(["readelf", "-d", LIB], capture_output=True, text=True).stdout
    needed = re.findall(r"NEEDED.*\[(.*)\]", out)
    assert not any("torch" in n or "c10" in n for n in needed)
    assert any("amdhip64" in n for n in needed)


def test_status_strings():
    from grouped_gemm_router_amd import binding as B
    for code, name in B.STATUS.items():
        assert B.status_string(code) == name


@pytest.mark.parametrize("args,expect", [
    ((64, 256, 128, 8, 2, "bf16"), 0),
    ((4096, 2048, 512, 256, 8, "bf16"), 0),
    ((8192, 4096, 1024, 512, 10, "mxfp8"), 0),
    ((0, 256, 128, 8, 2, "bf16"), 0),          # empty batch is valid
    ((64, 256, 128, 8, 9, "bf16"), 1),         # k > E
    ((64, 256, 128, 8, 0, "bf16"), 1),         # k < 1
    ((-1, 256, 128, 8, 2, "bf16"), 1),
    ((64, 0, 128, 8, 2, "bf16"), 1),
    ((64, 250, 128, 8, 2, "bf16"), 2),         # H not a multiple of 64
    ((64, 256, 100, 8, 2, "bf16"), 2),
    ((64, 192, 128, 8, 2, "mxfp8"), 2),        # MXFP8 needs multiples of 128
    ((64, 256, 128, 2048, 2, "bf16"), 2),      # E > 1024
    ((64, 256, 128, 64, 33, "bf16"), 2),       # k > 32
    ((2**28, 256, 128, 64, 8, "bf16"), 2),     # T*k >= 2^31
])
def test_validate_problem(args, expect):
    from grouped_gemm_router_amd import binding as B
    assert B.validate_problem(B.problem(*args)) == expect


def test_validate_problem_activation():
    from grouped_gemm_router_amd import binding as B
    assert B.validate_problem(B.problem(64, 256, 128, 8, 2)) == 0
    for act in ("swiglu", "geglu", "reglu", "relu2"):
        assert B.validate_problem(B.problem(64, 256, 128, 8, 2, activation=act)) == 0
    for act in ("swiglu_clamp", "swiglu_oai"):
        assert B.validate_problem(B.problem(64, 256, 128, 8, 2, activation=act, act_limit=7.0)) == 0
        assert B.validate_problem(B.problem(64, 256, 128, 8, 2, activation=act, act_limit=0.0)) == 1
        assert B.validate_problem(B.problem(64, 256, 128, 8, 2, activation=act, act_limit=float("nan"))) == 1
    p = B.problem(64, 256, 128, 8, 2)
    p.activation = 6
    assert B.validate_problem(p) == 1
    p.activation = -1
    assert B.validate_problem(p) == 1


def test_gate_pointers_optional_only_for_relu2():
    """The two-weight ReLU^2 expert takes NULL gate pointers; every gated activation needs them
    (argument errors, 1, come before the workspace check, 3, and the device check)."""
    import ctypes
    from grouped_gemm_router_amd import binding as B
    lib = B.lib
    v = ctypes.c_void_p(16)
    for act, expect in (("swiglu", 1), ("reglu", 1), ("relu2", 3)):
        p = B.problem(64, 256, 128, 8, 2, activation=act)
        # decode-sized problem (T <= 64): the missing workspace is reported once the pointers pass
        assert lib.moe_expert_mlp(ctypes.byref(p), v, v, v, None, v, v, None, None, None, v, v, None, 0,
                                  None) == expect, act
        ptrs = [v] * 15
        ptrs[7] = ptrs[11] = None                     # Wg_t, dW_gate
        assert lib.moe_backward(ctypes.byref(p), *ptrs, None, 0, None) == expect, act
    pm = B.problem(64, 256, 128, 8, 2, "mxfp8", activation="relu2")
    assert lib.moe_expert_mlp(ctypes.byref(pm), v, v, v, None, v, v, None, v, v, v, v, None, 0, None) == 3
    pm = B.problem(64, 256, 128, 8, 2, "mxfp8")
    assert lib.moe_expert_mlp(ctypes.byref(pm), v, v, v, v, v, v, None, v, v, v, v, None, 0, None) == 1


def test_workspace_sizes():
    from grouped_gemm_router_amd import binding as B
    p = B.problem(4096, 2048, 512, 256, 8)
    assert B.workspace_size(p, B.CALL_DISPATCH) >= 8 * 4 * 256 * 4
    assert B.workspace_size(p, B.CALL_EXPERT_MLP) == 0
    A, H, I = 4096 * 8, 2048, 512
    assert B.workspace_size(p, B.CALL_BACKWARD) >= A * I * 4 + A * 2 * I * 2 + A * I * 2 + A * H * 4
    pm = B.problem(8192, 4096, 1024, 512, 10, "mxfp8")
    assert B.workspace_size(pm, B.CALL_EXPERT_MLP) >= 8192 * 4096 + 81920 * 1024
    with pytest.raises(B.MoEError):
        B.workspace_size(pm, B.CALL_BACKWARD)          # backward is bf16 only
    with pytest.raises(B.MoEError):
        B.workspace_size(B.problem(64, 256, 128, 8, 9), B.CALL_DISPATCH)


def test_calls_reject_bad_arguments_before_touching_the_device():
    """Argument errors come back before the device check, so they are seen
    here even without a GPU (null pointers, k > E, small workspace)."""
    import ctypes
    from grouped_gemm_router_amd import binding as B
    lib = B.lib
    assert lib.moe_route(None, 4, 8, 2, None, None, None) == 1
    assert lib.moe_route(ctypes.c_void_p(16), 4, 8, 9, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == 1
    assert lib.moe_dispatch(ctypes.c_void_p(16), 4, 8, 2, ctypes.c_void_p(16), ctypes.c_void_p(16),
                            ctypes.c_void_p(16), ctypes.c_void_p(16), None, 0, None) == 3
    p = B.problem(64, 256, 128, 8, 2)
    assert lib.moe_expert_mlp(ctypes.byref(p), None, None, None, None, None, None, None, None, None, None,
                              None, None, 0, None) == 1
    # scales given for a bf16 problem
    v = ctypes.c_void_p(16)
    assert lib.moe_expert_mlp(ctypes.byref(p), v, v, v, v, v, v, v, v, v, v, v, None, 0, None) == 1
    pm = B.problem(64, 256, 128, 8, 2, "mxfp8")
    assert lib.moe_expert_mlp(ctypes.byref(pm), v, v, v, v, v, v, v, v, v, v, v, None, 0, None) == 3
    assert lib.moe_combine(v, v, v, 4, 2, 60, v, None) == 2
    assert lib.moe_mx_quantize(v, 4, 48, v, v, None) == 2
    assert lib.moe_pack_weights(v, 2, 100, 64, v, None) == 2
    assert lib.moe_backward(ctypes.byref(pm), *([v] * 15), None, 0, None) == 2
    # router backward: null pointers, k > E, E beyond the limit
    assert lib.moe_route_backward(None, v, v, 4, 8, 2, v, None) == 1
    assert lib.moe_route_backward(v, v, v, 4, 8, 9, v, None) == 1
    assert lib.moe_route_backward(v, v, v, 4, 2048, 2, v, None) == 2


def test_saved_pair_argument_checks():
    """moe_expert_mlp_save / moe_backward_saved: bf16 only (MXFP8 gives 2) and the saved
    projections are required (1), both reported before the device check."""
    import ctypes
    from grouped_gemm_router_amd import binding as B
    lib = B.lib
    v = ctypes.c_void_p(16)
    pm = B.problem(64, 256, 128, 8, 2, "mxfp8")
    assert lib.moe_expert_mlp_save(ctypes.byref(pm), *([v] * 9), None) == 2
    assert lib.moe_backward_saved(ctypes.byref(pm), *([v] * 16), v, 1 << 30, None) == 2
    p = B.problem(300, 256, 128, 8, 2)
    assert lib.moe_expert_mlp_save(ctypes.byref(p), *([v] * 8), None, None) == 1
    ptrs = [v] * 16
    ptrs[10] = None                                 # GU_rows
    assert lib.moe_backward_saved(ctypes.byref(p), *ptrs, v, 1 << 30, None) == 1


def test_empty_batch_accepts_null_token_arrays():
    """T = 0 is a valid problem: token-sized pointers may be NULL.  Calls that compute nothing
    return MOE_OK without touching the device; the others get past the argument checks and
    stop at the device check (no GPU here) or run (on a GPU)."""
    import ctypes
    from grouped_gemm_router_amd import binding as B
    lib = B.lib
    v = ctypes.c_void_p(16)
    assert lib.moe_route(None, 0, 8, 2, None, None, None) == 0
    assert lib.moe_route_backward(None, None, None, 0, 8, 2, None, None) == 0
    assert lib.moe_combine(None, None, None, 0, 2, 64, None, None) == 0
    p = B.problem(0, 256, 128, 8, 2)
    assert lib.moe_expert_mlp(ctypes.byref(p), None, None, v, v, v, v, None, None, None, None, None, None, 0,
                              None) == 0
    ptrs = [None] * 15
    ptrs[6] = v                                     # expert_offsets
    ptrs[7] = ptrs[8] = ptrs[9] = v                                  # packed weights
    ptrs[11] = ptrs[12] = ptrs[13] = v                               # dW_gate, dW_up, dW_down
    assert lib.moe_backward(ctypes.byref(p), *ptrs, None, 0, None) not in (1, 3)
    # the weights and the expert offsets are still required
    ptrs[8] = None
    assert lib.moe_backward(ctypes.byref(p), *ptrs, None, 0, None) == 1
    assert lib.moe_expert_mlp(ctypes.byref(p), None, None, None, v, v, v, None, None, None, None, None, None, 0,
                              None) == 1


def test_grouped_gemm_argument_checks():
    """moe_grouped_gemm: shape limits (2), null pointers and scale/dtype mismatches (1), and an
    empty row set that returns MOE_OK without touching the device."""
    import ctypes
    from grouped_gemm_router_amd import binding as B
    f = B.lib.moe_grouped_gemm
    v = ctypes.c_void_p(16)
    bf16, mx = B.DTYPE["bf16"], B.DTYPE["mxfp8"]
    assert f(bf16, v, 4, 0, 128, 64, None, None, v, None, None, None) == 0        # M = 0
    assert f(bf16, v, 4, 10, 100, 64, v, None, v, None, v, None) == 2             # N % 64
    assert f(bf16, v, 4, 10, 128, 96, v, None, v, None, v, None) == 2             # K % 64
    assert f(mx, v, 4, 10, 128, 64, v, v, v, v, v, None) == 2                     # MXFP8 K % 128
    assert f(bf16, v, 2048, 10, 128, 64, v, None, v, None, v, None) == 2          # E > 1024
    assert f(bf16, v, 4, 2 ** 25, 128, 128, v, None, v, None, v, None) == 2       # M * K >= 2^31
    assert f(bf16, None, 4, 10, 128, 64, v, None, v, None, v, None) == 1          # m_indptr
    assert f(bf16, v, 4, 10, 128, 64, None, None, v, None, v, None) == 1          # A
    assert f(bf16, v, 4, 10, 128, 64, v, v, v, None, v, None) == 1                # scales with bf16
    assert f(mx, v, 4, 10, 128, 128, v, None, v, v, v, None) == 1                 # missing SA
    assert f(7, v, 4, 10, 128, 64, v, None, v, None, v, None) == 1                # dtype
    assert f(bf16, v, 0, 10, 128, 64, v, None, v, None, v, None) == 1             # E = 0


def test_row_offset_limits():
    """Token rows (T*H bf16) and expert-major rows (T*k rows of up to 2I bf16) stay below the
    4 GiB the 32-bit byte offsets of the row loaders reach."""
    from grouped_gemm_router_amd import binding as B
    assert B.validate_problem(B.problem(2 ** 19, 2048, 256, 64, 2)) == 0          # T*H = 2^30, T*k*I = 2^28
    assert B.validate_problem(B.problem(2 ** 20, 2048, 64, 64, 1)) == 2           # T*H = 2^31
    assert B.validate_problem(B.problem(2 ** 18, 256, 1024, 64, 4)) == 2          # T*k*I = 2^30
    assert B.validate_problem(B.problem(2 ** 18, 256, 512, 64, 4)) == 0           # T*k*I = 2^29


def test_bench_refuses_several_gpus(monkeypatch, capsys):
    """bench.py measures one GPU: any other --gpus exits with status 2 and a
    message, before touching a device."""
    import sys
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err
