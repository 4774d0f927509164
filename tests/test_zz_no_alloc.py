"""The entry point that allocates nothing (moe_layer_forward_noalloc): its
buffers live in the library's static per-device scratch.  Through the C ABI
it must give what moe_layer_forward gives with a workspace (the same kernels,
so the same bits), on two calls in a row, the second with fewer rows."""
import sys

import pytest
import torch

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _both(W, x, accumulate=False):
    import quantized_routed_moe_router_amd as moe
    T, k, E = x.shape[0], W.n_expert_used, W.n_expert
    y0 = gu.dev(synth.activations(77, T, W.n_embd)) if accumulate else torch.zeros((T, W.n_embd), device="cuda")
    ya, ra = y0.clone(), moe.Routing(T, k, E)
    moe.layer_forward_noalloc(W, x, ya, routing=ra, accumulate=accumulate)
    yb, rb = y0.clone(), moe.Routing(T, k, E)
    ws = moe.alloc_workspace(W, T, moe.BF16 if x.dtype == torch.bfloat16 else moe.F32)
    moe.layer_forward(W, x, yb, ws, routing=rb, accumulate=accumulate)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
    for name in ("topk_idx", "topk_w", "count", "offset", "perm", "pos", "active", "n_active"):
        assert torch.equal(getattr(ra, name), getattr(rb, name)), name
    return ya


@pytest.mark.parametrize("T1,T2", [(8, 3), (16, 1)])
def test_noalloc_matches_layer_forward_flash_shape(T1, T2):
    # n_embd 4096, 16 experts of FFN width 2048, top-6, Q8_0 shared expert
    L = synth.make_layer(140, 0, D=4096, E=16, k=6, F=2048, Fs=2048)
    W = gu.upload(L)
    for T, seed in ((T1, 141), (T2, 142)):  # the second call has fewer rows
        _log("no-alloc flash shape T=%d" % T)
        x = gu.x_to_device(x=synth.activations(seed, T, 4096))
        _both(W, x)


@pytest.mark.parametrize("bf16", [False, True])
def test_noalloc_matches_layer_forward_mini(bf16):
    L = synth.make_layer(143, 0, D=512, E=32, k=4, F=256, Fs=128)
    W = gu.upload(L)
    for T, seed, acc in ((12, 144, False), (5, 145, True)):
        _log("no-alloc mini T=%d bf16=%s accumulate=%s" % (T, bf16, acc))
        xv = synth.activations(seed, T, 512)
        x = gu.x_to_device(x_bf16=synth.to_bf16_bits(xv)) if bf16 else gu.x_to_device(x=xv)
        _both(W, x, accumulate=acc)


def test_noalloc_matches_layer_forward_codebook_gate_up():
    # CB2 routed gate/up at n_embd 4096 (the codebook layers of the stack)
    L = synth.make_layer(148, 0, D=4096, E=16, k=6, F=512, Fs=2048, gate_fmt=synth.CB2, cb=synth.codebook(5))
    W = gu.upload(L)
    for T, seed in ((9, 149), (2, 150)):
        _log("no-alloc CB2 T=%d" % T)
        _both(W, gu.x_to_device(x=synth.activations(seed, T, 4096)))


def test_noalloc_rejects_many_rows():
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(146, 0, D=512, E=32, k=4, F=256, Fs=128)
    W = gu.upload(L)
    x = gu.x_to_device(x=synth.activations(147, 17, 512))
    y = torch.zeros((17, 512), device="cuda")
    with pytest.raises(moe.MoEError, match="few-row"):
        moe.layer_forward_noalloc(W, x, y)
