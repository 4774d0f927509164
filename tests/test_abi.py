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
            "moe_rmsnorm", "moe_dequant", "moe_version", "moe_count_selections", "moe_hotlist",
            "moe_read_stream", "moe_block_forward"} <= names
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
    # the activation codes of x and h must stay addressable with 32-bit
    # offsets: at n_embd 4096, k 6, FFN 2048 that is T*k*F*2 < 2^31
    assert _call_route(d, T=87382)[0] == -4
    assert _call_route(d, T=87381)[0] == -3  # accepted, then the 1 GiB workspace is short
    assert _call_route(d, T=2 ** 31 - 1)[0] == -4
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


# The Python binding checks every tensor before the library is called
# ("Understanding Dwarf Star" 3.7: validation fails early, nothing fails
# silently).  The library is replaced by a stub that fails the test if any
# entry point is reached.

class _NoLibrary:
    def __getattr__(self, name):
        raise AssertionError("the library was called (%s) despite a bad argument" % name)


def _cpu_layer(D=256, E=4, k=2, F=64, Fs=128):
    import torch

    import quantized_routed_moe_router_amd as moe
    u8 = dict(dtype=torch.uint8)
    return moe.LayerWeights(D, E, k, F, Fs, moe.Q2K, moe.Q2K, moe.Q2K, moe.Q8_0,
                            router_w=torch.zeros(E, D), gate=torch.zeros(E * F * D // 256 * 84, **u8),
                            up=torch.zeros(E * F * D // 256 * 84, **u8), down=torch.zeros(E * F * D // 256 * 84, **u8),
                            sh_gate=torch.zeros(Fs * D // 32 * 34, **u8), sh_up=torch.zeros(Fs * D // 32 * 34, **u8),
                            sh_down=torch.zeros(Fs * D // 32 * 34, **u8))


def _bad_call(case):
    import torch

    import quantized_routed_moe_router_amd as moe
    W = _cpu_layer()
    T, D = 3, W.n_embd
    x = torch.zeros(T, D)
    y = torch.zeros(T, D)
    ws = torch.zeros(1024, dtype=torch.uint8)
    r = moe.Routing(T, W.n_expert_used, W.n_expert, device="cpu")
    call = lambda: moe.layer_forward(W, x, y, ws, routing=r)
    if case == "x_width":
        x = torch.zeros(T, D + 256)
    elif case == "x_dtype":
        x = torch.zeros(T, D, dtype=torch.float64)
    elif case == "x_strided":
        x = torch.zeros(D, T).t()
    elif case == "x_1d":
        x = torch.zeros(T * D)
    elif case == "y_dtype":
        y = torch.zeros(T, D, dtype=torch.float64)
    elif case == "y_shape":
        y = torch.zeros(T + 1, D)
    elif case == "y_strided":
        y = torch.zeros(T, 2 * D)[:, ::2]
    elif case == "y_missing":
        y = None
    elif case == "ws_dtype":
        ws = torch.zeros(256, dtype=torch.int32)
    elif case == "routing_rows":
        r = moe.Routing(T + 1, W.n_expert_used, W.n_expert, device="cpu")
    elif case == "routing_dtype":
        r.topk_idx = r.topk_idx.long()
    elif case == "gate_bytes":
        W.gate = W.gate[:-84]
    elif case == "router_shape":
        W.router_w = torch.zeros(W.n_embd, W.n_expert)
    elif case == "on_cpu":
        pass  # every shape is right; the tensors are not on a GPU
    elif case == "route_without_routing":
        call = lambda: moe.route(W, x, None, ws)
    elif case == "ffn_without_routing":
        call = lambda: moe.expert_ffn(W, x, None, y, ws)
    elif case == "rmsnorm_gamma":
        call = lambda: moe.rmsnorm(x, torch.zeros(D - 1), y)
    elif case == "rmsnorm_out":
        call = lambda: moe.rmsnorm(x, torch.zeros(D), torch.zeros(T, D, dtype=torch.bfloat16))
    elif case == "dequant_src":
        call = lambda: moe.dequant(moe.Q2K, torch.zeros(83, dtype=torch.uint8), 256, torch.zeros(256))
    elif case == "dequant_out":
        call = lambda: moe.dequant(moe.Q2K, torch.zeros(84, dtype=torch.uint8), 256, torch.zeros(255))
    elif case == "counts_small":
        call = lambda: moe.count_selections(torch.zeros(2, 6, dtype=torch.int32), 256, 3,
                                            torch.zeros(3 * 256, dtype=torch.int64))
    elif case == "hotlist_order":
        call = lambda: moe.hotlist(torch.zeros(10, dtype=torch.int64), torch.zeros(9, dtype=torch.int32),
                                   torch.zeros(1, dtype=torch.int32))
    else:
        raise KeyError(case)
    return call


@pytest.mark.parametrize("case,exc,text", [
    ("x_width", ValueError, "n_embd"), ("x_dtype", TypeError, "x must be"), ("x_strided", ValueError, "contiguous"),
    ("x_1d", ValueError, "n_embd"), ("y_dtype", TypeError, "y must be"), ("y_shape", ValueError, "y must have"),
    ("y_strided", ValueError, "contiguous"), ("y_missing", TypeError, "y must be a torch.Tensor"),
    ("ws_dtype", TypeError, "ws must be"), ("routing_rows", ValueError, "routing.topk_idx"),
    ("routing_dtype", TypeError, "routing.topk_idx"), ("gate_bytes", ValueError, "gate holds"),
    ("router_shape", ValueError, "router_w"), ("on_cpu", ValueError, "CUDA device"),
    ("route_without_routing", ValueError, "routing"), ("ffn_without_routing", ValueError, "routing"),
    ("rmsnorm_gamma", ValueError, "gamma"), ("rmsnorm_out", TypeError, "out"), ("dequant_src", ValueError, "src"),
    ("dequant_out", ValueError, "out"), ("counts_small", ValueError, "counts"),
    ("hotlist_order", ValueError, "order"),
])
def test_binding_rejects_bad_tensors_before_the_library(monkeypatch, case, exc, text):
    import quantized_routed_moe_router_amd as moe
    call = _bad_call(case)
    monkeypatch.setattr(moe, "_lib", _NoLibrary())
    with pytest.raises(exc, match=text):
        call()


def test_read_stream_validates():
    import quantized_routed_moe_router_amd as moe
    err = ctypes.create_string_buffer(256)
    assert moe._lib.moe_read_stream(0x1000, 24, 0x2000, 4, None, err, 256) == -1      # not a multiple of 16
    assert moe._lib.moe_read_stream(0x1000, 32, 0x2000, 6, None, err, 256) == -1      # sink not a multiple of 4
    assert moe._lib.moe_read_stream(0x1008, 32, 0x2000, 4, None, err, 256) == -2      # misaligned
    assert moe._lib.moe_read_stream(None, 0, None, 4, None, err, 256) == 0            # nothing to read


def test_noalloc_entry_point_validates_before_touching_the_device():
    # the entry point without a workspace takes the few-row schedule only and
    # rejects shapes whose buffers exceed its static scratch, before any HIP call
    import quantized_routed_moe_router_amd as moe
    err = ctypes.create_string_buffer(256)
    f = moe._lib.moe_layer_forward_noalloc
    d = _desc()
    assert f(ctypes.byref(d), 0x80000, 17, 0, 0x100000, 0, None, None, err, 256) == -4  # beyond 16 rows
    assert b"few-row" in err.value
    big = _desc(n_expert=1024, n_expert_used=16, n_ff_exp=4096)  # 16 rows need more than the scratch
    assert f(ctypes.byref(big), 0x80000, 16, 0, 0x100000, 0, None, None, err, 256) == -3
    assert b"scratch" in err.value
    assert f(ctypes.byref(d), None, 0, 0, None, 0, None, None, err, 256) == 0  # T = 0: nothing to do
    assert f(ctypes.byref(d), 0x80008, 1, 0, 0x100000, 0, None, None, err, 256) == -2
    assert f(ctypes.byref(d), 0x80000, 1, 0, 0x100000, 4, None, None, err, 256) == -1  # unknown flag


def test_block_forward_validates():
    import quantized_routed_moe_router_amd as moe
    err = ctypes.create_string_buffer(256)
    f = moe._lib.moe_block_forward
    d = _desc()
    ws, n = 0x200000, 1 << 30
    assert f(ctypes.byref(d), None, 1e-6, 0x100000, 1, None, ws, n, None, err, 256) == -1  # no gamma
    assert f(ctypes.byref(d), 0x80008, 1e-6, 0x100000, 1, None, ws, n, None, err, 256) == -2  # misaligned gamma
    assert f(ctypes.byref(d), 0x80000, -1.0, 0x100000, 1, None, ws, n, None, err, 256) == -1  # eps < 0
    assert f(ctypes.byref(d), 0x80000, 1e-6, 0x100000, 1, None, ws, 16, None, err, 256) == -3  # workspace
    assert f(ctypes.byref(d), None, 1e-6, None, 0, None, ws, n, None, err, 256) == 0  # T = 0
