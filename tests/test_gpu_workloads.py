"""GPU parity at the full workload sizes (n_embd 4096, 256 experts, top-6,
FFN width 2048, Q8_0 shared expert), in the launch configuration the
benchmark times.  Routing and outputs are compared on every row; the oracle
evaluates the rows in chunks on the host cores."""
import os
import sys
import time

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def flash():
    t = time.time()
    L = synth.flash_layer()
    _log("flash layer generated in %.1f s" % (time.time() - t))
    return L, gu.upload(L)


def _run(wl, W):
    kw = dict(x_bf16=wl.x_bf16) if wl.x_bf16 is not None else dict(x=wl.x)
    L = wl.layers[0]
    _log("%s: T=%d on the GPU" % (wl.name, wl.T))
    y, r = gu.run_forward(W if L.router_bias is None else gu.upload_bias(W, L), gu.x_to_device(**kw))
    y = y.cpu().numpy()
    t = time.time()
    lg = oracle.logits(L, **kw)
    _, _, gap = oracle.topk(lg, L.n_expert_used, L.route_scale)
    y_ref, idx_ref, w_ref = gu.oracle_all_rows(L, **kw)
    _log("%s: oracle %.1f s on %d threads, min top-k margin %.3g" % (wl.name, time.time() - t,
                                                                      gu.oracle_workers(), gap.min()))
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)
    worst = gu.assert_close(y, y_ref)
    _log("%s: worst relative error %.3g over all %d rows" % (wl.name, worst, wl.T))


def test_decode_b1(flash):
    L, W = flash
    _run(synth.decode_b1(L), W)


def test_decode_b32_zipf(flash):
    L, W = flash
    _run(synth.decode_b32(L), W)


@pytest.mark.parametrize("T,zipf", [(8, False), (16, True)])
def test_decode_small_batches(flash, T, zipf):
    # the few-token path at full width with several tokens per bucket (the
    # Zipf router bias crowds the batch onto a few experts)
    import copy
    L, W = flash
    Lb = copy.copy(L)
    if zipf:
        Lb.router_bias = synth.zipf_bias(2, L.n_expert)
    wl = synth.Workload("decode_b%d%s" % (T, "_zipf" if zipf else ""), T, synth.F32, [Lb],
                        x=synth.activations(6, T, L.n_embd))
    _run(wl, W)


@pytest.mark.parametrize("E,k,Fs,accumulate", [(16, 4, 0, False), (12, 6, 2048, True), (8, 1, 2048, False),
                                                (6, 6, 0, True), (40, 3, 2048, False)])
def test_one_token_full_width(E, k, Fs, accumulate):
    # one token through full-width experts (n_embd 4096, FFN 2048) with fewer
    # slots than waves, with and without the shared expert, and adding into
    # y; two calls on one workspace and the four stages one by one give the
    # same bits, routing arrays included.
    import torch

    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(7, 0, D=4096, E=E, k=k, F=2048, Fs=Fs)
    x = synth.activations(8, 1, 4096)
    y0 = synth.activations(9, 1, 4096) if accumulate else np.zeros((1, 4096), np.float32)
    W = gu.upload(L)
    xd = gu.dev(x)
    _log("one token E=%d k=%d Fs=%d accumulate=%s on the GPU" % (E, k, Fs, accumulate))
    ws = moe.alloc_workspace(W, 1)
    outs = []
    for rep in range(2):  # the second call reuses the workspace (and its barrier counter)
        y = gu.dev(y0)
        r = moe.Routing(1, k, E)
        moe.layer_forward(W, xd, y, ws, routing=r, accumulate=accumulate)
        outs.append((y, r))
    ys = gu.dev(y0)
    rs = moe.Routing(1, k, E)
    for st in (1, 2, 3, 4):
        moe.layer_forward_stage(W, xd, ys, ws, st, routing=rs, accumulate=accumulate)
    torch.cuda.synchronize()
    for y, r in outs:
        assert torch.equal(y, ys)
        for name in ("topk_idx", "topk_w", "count", "offset", "perm", "pos", "active", "n_active"):
            assert torch.equal(getattr(r, name), getattr(rs, name)), name
    y_ref, _, _ = oracle.moe_forward(L, x=x)
    worst = gu.assert_close(outs[0][0].cpu().numpy(), y_ref + y0)
    _log("one token E=%d k=%d Fs=%d: worst relative error %.3g" % (E, k, Fs, worst))


@pytest.mark.parametrize("T", [1, 8])
def test_q4k_full_width(T):
    # Q4_K routed experts at full width (n_embd 4096, FFN 2048, top-6 of 16,
    # Q8_0 shared expert): the staged gate/up and down kernels take 144-byte
    # blocks (the down rows in batches of 8)
    L = synth.make_layer(12, 0, D=4096, E=16, k=6, F=2048, Fs=2048, gate_fmt=synth.Q4K, down_fmt=synth.Q4K)
    wl = synth.Workload("q4k_b%d" % T, T, synth.F32, [L], x=synth.activations(13, T, 4096))
    _run(wl, gu.upload(L))


def test_one_token_stages_and_repeats_are_bitwise_equal(flash):
    # the one-token schedule at full width: stages 1-4 one by one, and the
    # same call repeated on one workspace, give bitwise the same y and routing
    import torch

    import quantized_routed_moe_router_amd as moe
    L, W = flash
    x = gu.x_to_device(x=synth.activations(10, 1, L.n_embd))
    ws = moe.alloc_workspace(W, 1)
    r = moe.Routing(1, L.n_expert_used, L.n_expert)
    y = torch.zeros((1, L.n_embd), dtype=torch.float32, device="cuda")
    for st in (1, 2, 3, 4):
        moe.layer_forward_stage(W, x, y, ws, st, routing=r)
    outs = []
    for _ in range(3):
        y2 = torch.zeros_like(y)
        r2 = moe.Routing(1, L.n_expert_used, L.n_expert)
        moe.layer_forward(W, x, y2, ws, routing=r2)
        outs.append((y2, r2))
    torch.cuda.synchronize()
    for y2, r2 in outs:
        assert torch.equal(y, y2) and torch.equal(r.topk_idx, r2.topk_idx) and torch.equal(r.topk_w, r2.topk_w)
    y_ref, _, _ = oracle.moe_forward(L, x=x.cpu().numpy())
    gu.assert_close(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("T", [1, 3])
def test_exact_ties_across_waves_at_full_width(flash, T):
    # eight experts with the same router row and bias in every quarter of the
    # 256 (the one-token gate/up blocks select with their 4 waves, one quarter
    # each): the tied logits are the largest, so the top-6 are the six lowest
    # of the eight indices, and the cut falls inside the tie
    import copy

    import quantized_routed_moe_router_amd as moe
    L, W = flash
    tied = [5, 40, 64, 100, 129, 190, 200, 255]
    L2 = copy.copy(L)
    R = L.router_w.copy()
    for e in tied[1:]:
        R[e] = R[tied[0]]
    bias = np.zeros(L.n_expert, np.float32)
    bias[tied] = 40.0
    L2.router_w, L2.router_bias = R, bias
    W2 = copy.copy(W)
    W2.router_w, W2.router_bias = gu.dev(R), gu.dev(bias)
    x = synth.activations(30 + T, T, L.n_embd)
    y, r = gu.run_forward(W2, gu.x_to_device(x=x))
    y_ref, idx_ref, w_ref = gu.oracle_all_rows(L2, x=x)
    assert np.all(idx_ref == tied[:6])
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)
    worst = gu.assert_close(y.cpu().numpy(), y_ref)
    _log("ties across waves T=%d: worst relative error %.3g" % (T, worst))


def test_prefill_2048(flash):
    L, W = flash
    _run(synth.prefill_2048(L), W)


@pytest.fixture(scope="module")
def stack3():
    # three blocks of the 43-block stack at full width (n_embd 4096, FFN 2048,
    # top-6, CB2 gate/up, Q2K down, Q8_0 shared, RMSNorm weights), 16 experts
    # per layer to keep the codebook encoding short
    t = time.time()
    cb = synth.codebook(4)
    layers = [synth.stack_layer(l, cb, E=16) for l in range(3)]
    _log("stack layers generated in %.1f s" % (time.time() - t))
    return layers, [gu.upload(L) for L in layers]


@pytest.mark.parametrize("T", [3, 16, 24, 40])
def test_cb2_full_width_layer(stack3, T):
    # the codebook gate/up kernel at n_embd 4096 on its own, from a few tokens
    # to the decode schedule's 16 (several tokens per expert of 16); beyond 16
    # rows the batched kernels take the codebook blocks
    layers, Ws = stack3
    L = layers[0]
    x = synth.activations(120 + T, T, L.n_embd)
    _log("cb2 layer T=%d on the GPU" % T)
    y, r = gu.run_forward(Ws[0], gu.x_to_device(x=x))
    t = time.time()
    y_ref, idx_ref, w_ref = gu.oracle_all_rows(L, x=x)
    _log("cb2 layer T=%d: oracle %.1f s" % (T, time.time() - t))
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)
    worst = gu.assert_close(y.cpu().numpy(), y_ref)
    _log("cb2 layer T=%d: worst relative error %.3g" % (T, worst))


def _stack_on_gpu(Ws, x, block=False):
    # x <- x + MoE(RMSNorm(x)) layer by layer through the C ABI: rmsnorm, then
    # layer_forward accumulating into x, or (block) block_forward; returns
    # every layer's output
    import torch

    import quantized_routed_moe_router_amd as moe
    xd = gu.dev(x)
    xn = torch.empty_like(xd)
    ws = moe.alloc_workspace(Ws[0], x.shape[0])
    outs = []
    for W in Ws:
        if block:
            moe.block_forward(W, xd, ws)
        else:
            moe.rmsnorm(xd, W.gamma, xn, 1e-6)
            moe.layer_forward(W, xn, xd, ws, accumulate=True)
        outs.append(xd.cpu().numpy().copy())
    return outs


def _check_stack(layers, Ws, B, what):
    x = synth.stack43(B=B).x
    _log("%s B=%d: %d layers on the GPU" % (what, B, len(layers)))
    outs = _stack_on_gpu(Ws, x)
    t = time.time()
    # teacher forcing: each layer's output is compared with the oracle's on
    # the same input, so that errors do not compound
    ref = gu.oracle_stack(layers, x, teacher=[x] + outs[:-1])
    free = gu.oracle_stack(layers, x)
    _log("%s B=%d: oracle %.1f s" % (what, B, time.time() - t))
    for l in range(len(layers)):
        worst = gu.assert_close(outs[l], ref[l], what="layer %d output" % l)
        drift = float((np.abs(outs[l].astype(np.float64) - free[l]) / (1.0 + np.abs(free[l]))).max())
        _log("%s B=%d layer %d: worst relative error %.3g (teacher-forced), %.3g against the free-running oracle"
             % (what, B, l, worst, drift))


@pytest.mark.parametrize("B", [1, 8])
def test_stack_rmsnorm_residual_teacher_forced(stack3, B):
    layers, Ws = stack3
    _check_stack(layers, Ws, B, "stack of encoded 16-expert blocks")


@pytest.fixture(scope="module")
def stack4_flash():
    # four consecutive blocks of the 43-block stack at its own shape: 256
    # experts per layer, CB2 gate/up, Q2K down, Q8_0 shared, per-layer RMSNorm
    # weights; every block's fields drawn as random codes (the encoders would
    # take minutes per layer), which the oracle decodes like any other block
    t = time.time()
    cb = synth.codebook(4)
    layers = [synth.stack_layer_sampled(l, cb) for l in range(4)]
    _log("four 256-expert stack layers generated in %.1f s" % (time.time() - t))
    return layers, [gu.upload(L) for L in layers]


@pytest.mark.parametrize("B", [1, 8])
def test_stack_flash_shape_teacher_forced(stack4_flash, B):
    layers, Ws = stack4_flash
    _check_stack(layers, Ws, B, "stack of 256-expert blocks")


@pytest.mark.parametrize("B", [1, 8])
def test_block_forward_is_rmsnorm_then_layer_forward(stack4_flash, B):
    # block_forward (at one token: RMSNorm inside the first kernel, the
    # residual added by the last) gives the bits of rmsnorm followed by
    # layer_forward accumulating into x, layer after layer
    layers, Ws = stack4_flash
    x = synth.stack43(B=B).x
    composed = _stack_on_gpu(Ws, x)
    fused = _stack_on_gpu(Ws, x, block=True)
    for l in range(len(layers)):
        assert np.array_equal(fused[l].view(np.uint32), composed[l].view(np.uint32)), "layer %d" % l
    _log("block_forward B=%d: %d layers bitwise equal to rmsnorm + layer_forward" % (B, len(layers)))


def test_cb2_flash_shape_many_rows(stack4_flash):
    # the codebook layer at 256 experts with 32 rows: the batched kernels
    layers, Ws = stack4_flash
    L = layers[0]
    x = synth.activations(130, 32, L.n_embd)
    _log("cb2 256-expert layer T=32 on the GPU")
    y, r = gu.run_forward(Ws[0], gu.x_to_device(x=x))
    y_ref, idx_ref, w_ref = gu.oracle_all_rows(L, x=x)
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)
    worst = gu.assert_close(y.cpu().numpy(), y_ref)
    _log("cb2 256-expert layer T=32: worst relative error %.3g" % worst)
