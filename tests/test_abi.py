"""The C-ABI library: it loads, exports every entry point the header declares,
and its host-side validation answers without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mixture_experts_layer_27_amd", "libmoe_mi355x.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def b():
    if not os.path.exists(LIB):
        pytest.fail("library not built: run __graft_entry__.build()")
    from mixture_experts_layer_27_amd import binding
    return binding


def test_exports_every_declared_symbol(b):
    names = declared()
    assert len(names) >= 12
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert set(b.EXPORTS) == set(names)


def test_sizes_and_status_strings(b):
    s = b.make_shape(256, 128, 8, 2, 256, b.MOE_F32)
    assert b.max_rows(s) == 512
    assert b.plan_bytes(s) > 0
    assert b.workspace_bytes(s, b.MOE_WS_EXPERTS) >= 512 * 256 * 4
    assert b.workspace_bytes(s, b.MOE_WS_BACKWARD) > b.workspace_bytes(s, b.MOE_WS_EXPERTS)
    r = b.make_shape(1000, 256, 64, 8, 128, b.MOE_BF16, round_tile=128)
    assert b.max_rows(r) == 1000 * 8 + 64 * 64
    for code in range(5):
        assert b._lib.moe_status_str(code)


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), 1), (dict(k=9, E=16), 2), (dict(k=5, E=4), 1), (dict(E=300), 2), (dict(d=100), 2),
    (dict(d_ff=96), 2), (dict(act=7), 1), (dict(round_tile=3), 1), (dict(T=(1 << 20) + 1), 2),
    (dict(gate_mode=2), 1), (dict(capacity_factor=-1.0), 1), (dict(lb_coef=float("nan")), 1),
    (dict(z_coef=float("inf")), 1), (dict(capacity_factor=1.0, round_tile=128), 2),
])
def test_shape_validation(b, kw, code):
    base = dict(T=64, d=128, E=8, k=2, d_ff=128, act=b.MOE_BF16, gemm=None, round_tile=0)
    base.update(kw)
    s = b.make_shape(**base)
    assert b.plan_bytes(s) == 0 and b.max_rows(s) == -1
    plan = b.MoePlan()
    blob = ctypes.c_void_p(1 << 20)   # host address: never dereferenced on the error path
    got = b._lib.moe_plan_init(ctypes.byref(s), blob, 1 << 30, ctypes.byref(plan))
    assert got == code


def test_argument_errors_return_before_launch(b):
    s = b.make_shape(64, 128, 8, 2, 128, b.MOE_BF16)
    plan = b.MoePlan()
    fake = ctypes.c_void_p(1 << 20)
    assert b._lib.moe_plan_init(ctypes.byref(s), fake, 16, ctypes.byref(plan)) == 3      # blob too small
    assert b._lib.moe_plan_init(ctypes.byref(s), ctypes.c_void_p((1 << 20) + 8), 1 << 30, ctypes.byref(plan)) == 1
    assert b._lib.moe_plan_init(ctypes.byref(s), fake, 1 << 30, ctypes.byref(plan)) == 0
    # null inputs, misaligned pointers, missing workspace: rejected on the host
    assert b._lib.moe_route(ctypes.byref(s), None, fake, None, None, ctypes.byref(plan), None, 0, None) == 1
    assert b._lib.moe_permute(ctypes.byref(s), ctypes.c_void_p((1 << 20) + 4), ctypes.byref(plan), fake, None) == 1
    assert b._lib.moe_grouped_gemm_swiglu(ctypes.byref(s), fake, fake, fake, ctypes.byref(plan), fake, fake,
                                          fake, 0, None) == 3
    assert b._lib.moe_backward(ctypes.byref(s), fake, fake, fake, fake, ctypes.byref(plan), fake, None, None, fake, fake,
                               fake, fake, fake, None, None, fake, 0, None) == 3
    assert b._lib.moe_round_tokens(ctypes.byref(s), ctypes.byref(plan), None, 0, None) == 1   # rounding off
    assert b._lib.moe_quantize_mx(fake, 4, 48, 1, fake, fake, None) == 1                      # cols % 32
    assert b._lib.moe_quantize_mx(fake, 96, 64, 0, fake, fake, None) == 1                     # rows % 64
    assert b._lib.moe_quantize_mx(fake, 64, 64, 2, fake, fake, None) == 1                     # k_axis
    empty = b.MoePlan()
    assert b._lib.moe_unpermute_combine(ctypes.byref(s), fake, ctypes.byref(empty), fake, None) == 1


def test_trace_validation_returns_before_launch(b):
    """A trace whose events are missing is rejected on the host (nothing launched)."""
    s = b.make_shape(64, 128, 8, 2, 128, b.MOE_BF16)
    plan = b.MoePlan()
    fake = ctypes.c_void_p(1 << 20)
    assert b._lib.moe_plan_init(ctypes.byref(s), fake, 1 << 30, ctypes.byref(plan)) == 0
    handles = (ctypes.c_void_p * 4)()                      # all NULL
    tr = b.MoeTrace(ctypes.cast(handles, ctypes.POINTER(ctypes.c_void_p)), 4, 0)
    assert b._lib.moe_grouped_gemm_swiglu_traced(ctypes.byref(s), fake, fake, fake, ctypes.byref(plan), fake, fake,
                                                 fake, 1 << 30, None, ctypes.byref(tr)) == 1
    assert b._lib.moe_backward_traced(ctypes.byref(s), fake, fake, fake, fake, ctypes.byref(plan), fake, None, None,
                                      fake, fake, fake, fake, fake, None, None, fake, 1 << 40, None,
                                      ctypes.byref(tr)) == 1
    neg = b.MoeTrace(ctypes.cast(handles, ctypes.POINTER(ctypes.c_void_p)), -1, 0)
    assert b._lib.moe_grouped_gemm_swiglu_gather_traced(ctypes.byref(s), fake, fake, fake, ctypes.byref(plan), fake,
                                                        fake, fake, 1 << 30, None, ctypes.byref(neg)) == 1
    assert tr.count == 0


def test_noalloc_rejects_problems_past_its_scratch(b):
    """The no-allocation expert FFN refuses, on the host, a problem whose workspace
    exceeds the library's device scratch (nothing is launched)."""
    fake = ctypes.c_void_p(1 << 20)
    s = b.make_shape(16384, 2048, 128, 4, 1024, b.MOE_BF16)      # A alone is 128 MiB
    assert b.workspace_bytes(s, b.MOE_WS_EXPERTS) > b.NOALLOC_SCRATCH_BYTES
    plan = b.MoePlan()
    assert b._lib.moe_plan_init(ctypes.byref(s), fake, 1 << 40, ctypes.byref(plan)) == 0
    assert b._lib.moe_grouped_gemm_swiglu_noalloc(ctypes.byref(s), fake, fake, fake, ctypes.byref(plan), fake, fake,
                                                  None) == 3
    small = b.make_shape(64, 128, 8, 2, 128, b.MOE_BF16)
    assert b.workspace_bytes(small, b.MOE_WS_EXPERTS) <= b.NOALLOC_SCRATCH_BYTES
    assert b._lib.moe_grouped_gemm_swiglu_noalloc(ctypes.byref(small), None, fake, fake, ctypes.byref(plan), fake,
                                                  fake, None) == 1


def test_weight_codes_validation_returns_before_launch(b):
    """The MXFP8 weight-code calls refuse other GEMM types, a short workspace and a
    bad x_gathered flag on the host (nothing launched)."""
    fake = ctypes.c_void_p(1 << 20)
    bf = b.make_shape(64, 128, 8, 2, 128, b.MOE_BF16)
    mx = b.make_shape(64, 128, 8, 2, 128, b.MOE_BF16, gemm=b.MOE_MXFP8)
    plan = b.MoePlan()
    assert b._lib.moe_plan_init(ctypes.byref(mx), fake, 1 << 30, ctypes.byref(plan)) == 0
    assert b._lib.moe_quantize_weights_mx(ctypes.byref(bf), fake, fake, fake, 1 << 30, None) == 2
    assert b._lib.moe_quantize_weights_mx(ctypes.byref(mx), fake, fake, fake, 16, None) == 3
    assert b._lib.moe_quantize_weights_mx(ctypes.byref(mx), None, fake, fake, 1 << 30, None) == 1
    wc = b._lib.moe_grouped_gemm_swiglu_wcodes
    assert wc(ctypes.byref(bf), fake, 1, ctypes.byref(plan), fake, fake, fake, 1 << 30, None, None) == 2
    assert wc(ctypes.byref(mx), fake, 2, ctypes.byref(plan), fake, fake, fake, 1 << 30, None, None) == 1
    assert wc(ctypes.byref(mx), fake, 1, ctypes.byref(plan), fake, fake, fake, 16, None, None) == 3
    assert wc(ctypes.byref(mx), None, 0, ctypes.byref(plan), fake, fake, fake, 1 << 30, None, None) == 1


def test_combine_entry_validation_returns_before_launch(b):
    """The combine-in-GEMM2 call refuses fp32 and MXFP8 GEMMs, a bad x_gathered
    flag and a short workspace on the host (nothing launched)."""
    fake = ctypes.c_void_p(1 << 20)
    bf = b.make_shape(64, 128, 8, 2, 128, b.MOE_BF16)
    f32 = b.make_shape(64, 128, 8, 2, 128, b.MOE_F32)
    mx = b.make_shape(64, 128, 8, 2, 128, b.MOE_BF16, gemm=b.MOE_MXFP8)
    assert b.workspace_bytes(bf, b.MOE_WS_EXPERTS_COMBINE) >= (b.workspace_bytes(bf, b.MOE_WS_EXPERTS)
                                                              + b.max_rows(bf) * (128 * 2 + 4))
    plan = b.MoePlan()
    assert b._lib.moe_plan_init(ctypes.byref(bf), fake, 1 << 30, ctypes.byref(plan)) == 0
    cb = b._lib.moe_grouped_gemm_swiglu_combine
    args = lambda flag, n: (fake, flag, fake, fake, ctypes.byref(plan), fake, fake, fake, n, None, None)
    assert cb(ctypes.byref(f32), *args(1, 1 << 30)) == 2
    assert cb(ctypes.byref(mx), *args(1, 1 << 30)) == 2
    assert cb(ctypes.byref(bf), *args(3, 1 << 30)) == 1
    assert cb(ctypes.byref(bf), *args(1, 16)) == 3
    assert cb(ctypes.byref(bf), None, 1, fake, fake, ctypes.byref(plan), fake, fake, fake, 1 << 30, None, None) == 1


def test_ref_stream_validation(b):
    fake = ctypes.c_void_p(1 << 20)
    assert b._lib.moe_ref_stream(fake, fake, 15, 2, None) == 1                 # not a multiple of 16
    assert b._lib.moe_ref_stream(fake, fake, 1 << 20, 4, None) == 1            # mode
    assert b._lib.moe_ref_stream(None, fake, 1 << 20, 2, None) == 1            # copy without a source
    assert b._lib.moe_ref_stream(fake, ctypes.c_void_p((1 << 20) + 8), 64, 1, None) == 1   # misaligned
