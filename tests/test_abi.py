"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src))
    return names


def test_exports_every_declared_symbol():
    import quantized_routed_moe_router_amd as moe
    names = _declared()
    assert {"moe_route", "moe_expert_ffn", "moe_layer_forward", "moe_layer_forward_stage", "moe_workspace_size",
            "moe_rmsnorm", "moe_dequant", "moe_version", "moe_count_selections", "moe_hotlist"} <= names
    for n in names:
        assert hasattr(moe._lib, n), n
    assert moe.version().startswith("moe-gfx950")


def _desc(**kw):
    import quantized_routed_moe_router_amd as moe
    base = dict(n_embd=4096, n_expert=256, n_expert_used=6, n_ff_exp=2048, n_ff_shared=2048,
                gate_type=moe.Q2K, up_type=moe.Q2K, down_type=moe.Q2K, shared_type=moe.Q8_0,
                router_w=0x10000, router_bias=None, route_scale=1.0, gate=0x20000, up=0x30000, down=0x40000,
                sh_gate=0x50000, sh_up=0x60000, sh_down=0x70000, codebook=None)
    base.update(kw)
    return moe.LayerDesc(*[base[f] for f, _ in moe.LayerDesc._fields_])


def _call_route(d, T=1, x=0x80000, ws=0x90000, ws_bytes=1 << 30, x_type=0):
    import quantized_routed_moe_router_amd as moe
    r = moe.RoutingStruct(*([0xA0000] * 8))
    err = ctypes.create_string_buffer(256)
    rc = moe._lib.moe_route(ctypes.byref(d), x, T, x_type, ctypes.byref(r), ws, ws_bytes, None, err, 256)
    return rc, err.value.decode()


def test_workspace_size():
    import quantized_routed_moe_router_amd as moe
    d = _desc()
    n1 = moe._lib.moe_workspace_size(ctypes.byref(d), 1, 0)
    n2048 = moe._lib.moe_workspace_size(ctypes.byref(d), 2048, 1)
    assert 0 < n1 < n2048
    assert moe._lib.moe_workspace_size(None, 1, 0) == 0
    assert moe._lib.moe_workspace_size(ctypes.byref(_desc(n_expert_used=300)), 1, 0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(n_expert_used=7, n_expert=6), -4),       # k > E
    (dict(n_expert_used=17, n_expert=64), -4),     # k > 16
    (dict(n_expert=2000), -4),                      # E > 1024
    (dict(n_embd=4000), -4),                        # D % 256
    (dict(n_ff_exp=192), -4),                       # F/64 not a power of two
    (dict(gate_type=1), -4),                        # not a block format
    (dict(up_type=4), -4),                          # gate != up
    (dict(gate_type=4, up_type=4), -1),             # CB2 without codebook
    (dict(gate=None), -1),
    (dict(sh_down=None), -1),
    (dict(router_w=0x10004), -2),                   # misaligned
    (dict(n_embd=0), -1),
])
def test_bad_descriptors_are_rejected(kw, code):
    rc, msg = _call_route(_desc(**kw))
    assert rc == code and msg


def test_bad_calls_are_rejected():
    d = _desc()
    assert _call_route(d, T=-1)[0] == -1
    assert _call_route(d, x=None)[0] == -1
    assert _call_route(d, x=0x80008)[0] == -2
    assert _call_route(d, ws_bytes=100)[0] == -3
    assert _call_route(d, ws=None)[0] == -3
    assert _call_route(d, x_type=3)[0] == -4
    # T = 0 is a valid no-op and touches nothing
    assert _call_route(d, T=0, x=None, ws=None, ws_bytes=0)[0] == 0


def test_other_entry_points_validate():
    import quantized_routed_moe_router_amd as moe
    err = ctypes.create_string_buffer(256)
    assert moe._lib.moe_dequant(1, 0x1000, 256, None, 0, 0x2000, None, err, 256) == -4
    assert moe._lib.moe_dequant(2, 0x1000, 255, None, 0, 0x2000, None, err, 256) == -1
    assert moe._lib.moe_dequant(4, 0x1000, 256, None, 0, 0x2000, None, err, 256) == -1
    assert moe._lib.moe_dequant(2, 0x1000, 0, None, 0, 0x2000, None, err, 256) == 0
    assert moe._lib.moe_rmsnorm(0x1000, 0x2000, ctypes.c_float(1e-6), -1, 64, 0x3000, None, err, 256) == -1
    assert moe._lib.moe_rmsnorm(None, None, ctypes.c_float(1e-6), 0, 64, None, None, err, 256) == 0
    d = _desc()
    r = moe.RoutingStruct(*([0xA0000] * 8))
    assert moe._lib.moe_expert_ffn(ctypes.byref(d), 0x80000, 1, 0, ctypes.byref(r), 0x100004, 0, 0x90000, 1 << 30,
                                   None, err, 256) == -2
    assert moe._lib.moe_expert_ffn(ctypes.byref(d), 0x80000, 1, 0, ctypes.byref(r), 0x100000, 8, 0x90000, 1 << 30,
                                   None, err, 256) == -1
    assert moe._lib.moe_layer_forward(ctypes.byref(d), 0x80000, 1, 0, None, 0, None, 0x90000, 1 << 30, None,
                                      err, 256) == -1
    for stage in (0, 6):
        assert moe._lib.moe_layer_forward_stage(ctypes.byref(d), 0x80000, 1, 0, 0x100000, 0, None, stage, 0x90000,
                                                1 << 30, None, err, 256) == -1


def test_hotlist_and_counts_validate_before_enqueue():
    import quantized_routed_moe_router_amd as moe
    err = ctypes.create_string_buffer(256)
    assert moe._lib.moe_hotlist(None, 16385, None, None, None, err, 256) == -1
    assert b"16384" in err.value
    assert moe._lib.moe_hotlist(None, 0, None, None, None, err, 256) == 0  # nothing to sort
    assert moe._lib.moe_count_selections(None, 4, 0, 8, 0, None, None, err, 256) == -1
    assert moe._lib.moe_count_selections(None, 0, 6, 8, 0, None, None, err, 256) == 0  # T = 0
    assert moe._lib.moe_count_selections(None, 1, 6, 8, 0, None, None, err, 256) == -1  # pointers unset
