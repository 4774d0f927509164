"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Integer results (indices, bucketing, decoded weights)
must match bit for bit; fp32 outputs within |gpu-ref| <= 2e-3 (1+|ref|)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _bf16_bits_of(f32):
    u = np.asarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", [synth.Q2K, synth.Q8_0, synth.CB2, synth.Q4K])
def test_dequant_bit_exact(fmt):
    import quantized_routed_moe_router_amd as moe
    cb = synth.codebook(4)
    n = 256 * 96
    b = synth.expert_tensor(fmt, 7, 0, 3, 1, n // 256, 256, codebook=cb)
    ref = oracle.dequant(fmt, b, n, codebook=cb)
    src = gu.dev(b)
    cbd = gu.dev(cb) if fmt == synth.CB2 else None
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    moe.dequant(fmt, src, n, out, codebook=cbd)
    outb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    moe.dequant(fmt, src, n, outb, codebook=cbd)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(outb.cpu().view(torch.int16).numpy().view(np.uint16), _bf16_bits_of(ref))
    # code-sampled blocks (all fields uniform) decode the same way
    b2 = synth.sampled_tensor(fmt, 8, 0, 3, 1, n // 256, 256, codebook=cb)
    moe.dequant(fmt, gu.dev(b2), n, out, codebook=cbd)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle.dequant(fmt, b2, n, codebook=cb).view(np.uint32))


def _check_layer(L, T, seed, bf16=False, rows=None):
    x = synth.activations(seed, T, L.n_embd)
    kw = dict(x_bf16=synth.to_bf16_bits(x)) if bf16 else dict(x=x)
    y_ref, idx_ref, w_ref = oracle.moe_forward(L, rows=rows, **kw)
    W = gu.upload(L)
    y, r = gu.run_forward(W, gu.x_to_device(**kw))
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)
    yg = y.cpu().numpy()
    sel = slice(None) if rows is None else rows
    return gu.assert_close(yg[sel], y_ref[sel]), W, y


@pytest.mark.parametrize("T", [1, 5, 37])
def test_q4k_routed_layers(T):
    # Q4_K routed gate/up/down with a Q8_0 shared expert: one token and a few
    # (the staged decode kernels) and a batch (the batched kernels)
    L = synth.make_layer(110, 0, D=512, E=32, k=4, F=256, Fs=128, gate_fmt=synth.Q4K, down_fmt=synth.Q4K)
    _check_layer(L, T, 111 + T)


def test_tiny_workload():
    wl = synth.tiny()
    _check_layer(wl.layers[0], wl.T, 0)


@pytest.mark.parametrize("T", [1, 5, 37])
@pytest.mark.parametrize("shared", [True, False])
def test_mini_layers_several_tiles(T, shared):
    L = synth.make_layer(50 + T, 0, D=512, E=32, k=4, F=256, Fs=128 if shared else 0)
    _check_layer(L, T, 60 + T)


@pytest.mark.parametrize("T", [3, 33])
def test_bf16_small(T):
    L = synth.make_layer(70, 0, D=512, E=32, k=4, F=256, Fs=128)
    _check_layer(L, T, 71, bf16=True)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("D,F,E,k,T,Fs", [
    (512, 512, 8, 2, 150, 256),   # 1- and 2-subtile tiles with ragged rows
    (256, 256, 4, 2, 300, 0),     # several tiles per expert; one super-block column
    (1024, 256, 16, 6, 57, 128),
    (512, 256, 32, 4, 24, 128),   # at most 32 rows: the 4-wave variant, two blocks per compute unit
    (512, 512, 4, 2, 32, 0),      # a bucket of all 32 rows
])
def test_many_rows_matrix_cores(D, F, E, k, T, Fs, bf16):
    # batches beyond the decode schedule run as grouped GEMMs on the matrix
    # cores, bf16 rows (h in bf16, atomic combine) and fp32 rows (h in fp32,
    # per-pair rows gathered in slot order); outputs within tolerance of the
    # oracle in the same mode
    L = synth.make_layer(74 + T, 0, D=D, E=E, k=k, F=F, Fs=Fs)
    worst, _, _ = _check_layer(L, T, 75 + T, bf16=bf16)
    print("%s D=%d F=%d E=%d k=%d T=%d: worst relative error %.3g" % ("bf16" if bf16 else "fp32", D, F, E, k, T,
                                                                        worst))


def test_shared_expert_matrix_cores_full_width():
    # the shared expert of fp32 rows as int8 matrix-core GEMMs at its full
    # width (n_embd 4096, n_ff_shared 2048): a ragged second 16-row tile, a
    # second pass over the rows, and an all-zero row (its scale is 0)
    L = synth.make_layer(120, 0, D=4096, E=8, k=2, F=256, Fs=2048)
    T = 35
    x = synth.activations(121, T, 4096)
    x[7] = 0.0
    y_ref, idx_ref, w_ref = oracle.moe_forward(L, x=x)
    W = gu.upload(L)
    y, r = gu.run_forward(W, gu.x_to_device(x=x))
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)
    worst = gu.assert_close(y.cpu().numpy(), y_ref)
    print("fp32 shared expert at full width, T=%d: worst relative error %.3g" % (T, worst))


def test_bf16_many_rows_accumulate():
    L = synth.make_layer(76, 0, D=512, E=8, k=2, F=512, Fs=256)
    x = synth.activations(77, 40, 512)
    xb = synth.to_bf16_bits(x)
    y_ref, _, _ = oracle.moe_forward(L, x_bf16=xb)
    W = gu.upload(L)
    y0 = torch.full((40, 512), -0.5, dtype=torch.float32, device="cuda")
    y, _ = gu.run_forward(W, gu.x_to_device(x_bf16=xb), accumulate=True, y0=y0)
    gu.assert_close(y.cpu().numpy(), y_ref - np.float32(0.5))


def test_cb2_gate_up_layer():
    cb = synth.codebook(4)
    L = synth.make_layer(72, 0, D=1024, E=16, k=6, F=512, Fs=256, gate_fmt=synth.CB2, cb=cb)
    _check_layer(L, 9, 73)


def test_cb2_codebook_range_ends():
    # the codebook gate/up kernel at n_embd 4096 with codebook values at the
    # ends of the range it takes, [-127, 127] (its bytewise negation is
    # carry-free there), and every block's indices redrawn over the four
    # extreme entries so that they are used throughout; every block scale is
    # set so that the weights keep the magnitude of N(0, 0.02) draws
    cb = np.clip(synth.codebook(4).astype(np.int32) * 15, -127, 127).astype(np.int8)
    cb[0] = [127, -127, 127, -127, 127, -127, 127, -127]
    cb[1] = -127
    cb[2] = 127
    cb[3] = [0, 127, -127, 0, 1, -1, 126, -126]
    L = synth.make_layer(130, 0, D=4096, E=8, k=2, F=128, Fs=0, gate_fmt=synth.CB2, cb=cb)
    for i, name in enumerate(("gate", "up")):
        g = np.ascontiguousarray(getattr(L, name)).copy()
        blocks = g.reshape(-1, 66)
        u = synth.uniform(131 + i, 0, synth.TAG_X, 0, blocks.shape[0] * 32)
        blocks[:, 2:34] = (u * 4).astype(np.uint8).reshape(-1, 32)
        blocks[:, 0:2] = np.array([1.5e-4], dtype=np.float16).view(np.uint8)
        setattr(L, name, g)
    worst, _, _ = _check_layer(L, 3, 133)
    print("cb2 range ends: worst relative error %.3g" % worst)


@pytest.mark.parametrize("E,k", [(1, 1), (6, 6), (16, 1)])
def test_degenerate_routings(E, k):
    L = synth.make_layer(80 + E, 0, D=256, E=E, k=k, F=128, Fs=64)
    _check_layer(L, 7, 81)


def test_exact_ties_go_to_lower_index():
    L = synth.make_layer(90, 0, D=256, E=16, k=3, F=128, Fs=0)
    W = L.router_w.copy()
    W[12] = W[3]
    W[9] = W[3]
    L.router_w = W
    bias = np.zeros(16, np.float32)
    bias[[3, 9, 12]] = 40.0
    L.router_bias = bias
    _check_layer(L, 6, 91)
    _, idx, _ = oracle.moe_forward(L, x=synth.activations(91, 6, 256))
    assert np.all(idx == [3, 9, 12])


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("T", [40, 128, 203])
def test_route_many_rows_matrix_cores(T, bf16):
    # beyond 16 rows the logits run on the fp64 matrix cores (four waves per
    # tile below 128 rows, one from 128 on): ragged token and expert tiles
    # (E = 40 is 2.5 tiles of 16), a Zipf bias, fp32 and bf16 x; indices and
    # bucketing bit-exact, weights within tolerance
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(94, 0, D=512, E=40, k=6, F=128, Fs=0)
    L.router_bias = synth.zipf_bias(95, 40)
    x = synth.activations(96 + T, T, 512)
    kw = dict(x_bf16=synth.to_bf16_bits(x)) if bf16 else dict(x=x)
    idx_ref, w_ref, gap = oracle.route(L, **kw)
    print("route T=%d bf16=%s: smallest k/k+1 logit gap %.3g" % (T, bf16, float(np.min(gap))))
    W = gu.upload(L)
    xd = gu.x_to_device(**kw)
    ws = moe.alloc_workspace(W, T, moe.BF16 if bf16 else moe.F32)
    r = moe.Routing(T, L.n_expert_used, L.n_expert)
    moe.route(W, xd, r, ws)
    torch.cuda.synchronize()
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)


@pytest.mark.parametrize("T,E,k,D,bias", [(128, 256, 6, 4096, False), (203, 40, 6, 1024, True),
                                          (300, 200, 8, 2048, True), (160, 256, 6, 1024, False),
                                          (129, 64, 1, 4096, True)])
def test_route_two_pass_bf16(T, E, k, D, bias):
    # 128 or more bf16 rows: the logits are first bounded on the bf16 matrix
    # cores (three-part weights, fp32 sums), then the experts that can still
    # reach the top k are computed again exactly.  Exact ties (four copies of
    # one enlarged router row, so they reach the top k often), a near tie (a
    # fifth copy with one weight changed in its last bit), ragged token and
    # expert tiles, k = 1 and 8, a Zipf bias, a zero row (all logits equal):
    # indices and bucketing bit-exact against the fp64 oracle, weights within
    # tolerance
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(120 + T, 0, D=D, E=E, k=k, F=256, Fs=0)
    rw = np.array(L.router_w, dtype=np.float32).reshape(E, D)
    base = E // 3
    rw[base] *= np.float32(3.0)
    for e in (base + 1, base + 2, E - 1):
        rw[e] = rw[base]
    near = rw[base].copy()
    near[D // 2] = np.nextafter(near[D // 2], np.float32(np.inf))
    rw[base + 3] = near
    L.router_w = rw.reshape(np.shape(L.router_w))
    if bias:
        L.router_bias = synth.zipf_bias(121 + T, E)
    x = synth.activations(122 + T, T, D)
    x[5] = 0.0  # every logit equal (the bias alone): every expert is a candidate
    xb = synth.to_bf16_bits(x)
    idx_ref, w_ref, gap = oracle.route(L, x_bf16=xb)
    n_tied = int(np.sum(np.isin(idx_ref, [base, base + 1, base + 2, base + 3, E - 1])))
    print("two-pass route T=%d E=%d D=%d: %d selections among the tied rows, smallest k/k+1 gap %.3g"
          % (T, E, D, n_tied, float(np.min(gap))))
    assert n_tied > 0
    W = gu.upload(L)
    xd = gu.x_to_device(x_bf16=xb)
    ws = moe.alloc_workspace(W, T, moe.BF16)
    r = moe.Routing(T, k, E)
    moe.route(W, xd, r, ws)
    torch.cuda.synchronize()
    gu.check_routing(r, idx_ref, w_ref, E)


@pytest.mark.parametrize("T,E,k,D", [(17, 1024, 1, 512), (170, 64, 6, 512), (256, 8, 4, 512), (64, 512, 16, 512),
                                     (33, 300, 3, 512), (171, 64, 6, 512), (33, 256, 6, 4096), (100, 64, 8, 2048),
                                     (17, 16, 2, 1024), (127, 200, 8, 4096)])
def test_route_one_block_sort_bounds(T, E, k, D):
    # 17 to 1024 pairs: one block selects every row's top k and sorts the
    # pairs (16 waves of 64 pairs): the largest expert count (ten key bits),
    # exactly 1024 pairs with every expert active, the largest k, an expert
    # count that is no power of two, one pair over the bound (the many-pair
    # sort instead), and below 128 rows with n_embd 1024 to 4096 the router's
    # reduction split over 2, 4 and 8 blocks whose partial sums the selection
    # adds (ragged token and expert tiles at 127 rows and 200 experts)
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(130 + T, 0, D=D, E=E, k=k, F=64, Fs=0)
    L.router_bias = synth.zipf_bias(131, E)
    x = synth.activations(132 + T, T, D)
    idx_ref, w_ref, gap = oracle.route(L, x=x)
    W = gu.upload(L)
    ws = moe.alloc_workspace(W, T)
    r = moe.Routing(T, k, E)
    moe.route(W, gu.x_to_device(x=x), r, ws)
    torch.cuda.synchronize()
    print("route T=%d E=%d k=%d: %d active, smallest k/k+1 gap %.3g" % (T, E, k, int(r.n_active.cpu()[0]),
                                                                        float(np.min(gap))))
    gu.check_routing(r, idx_ref, w_ref, E)


def test_route_scale_and_accumulate():
    L = synth.make_layer(92, 0, D=512, E=32, k=4, F=256, Fs=128)
    L.route_scale = 1.5
    x = synth.activations(93, 4, 512)
    y_ref, _, _ = oracle.moe_forward(L, x=x)
    W = gu.upload(L)
    y0 = torch.full((4, 512), 0.25, dtype=torch.float32, device="cuda")
    y, _ = gu.run_forward(W, gu.x_to_device(x=x), accumulate=True, y0=y0)
    gu.assert_close(y.cpu().numpy(), y_ref + np.float32(0.25))


def test_zero_rows_is_a_no_op():
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(94, 0, D=256, E=16, k=2, F=128, Fs=0)
    W = gu.upload(L)
    x = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    y = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    moe.layer_forward(W, x, y, ws)
    torch.cuda.synchronize()


def test_run_twice_is_bitwise_identical_and_batch_invariant():
    L = synth.make_layer(95, 0, D=512, E=32, k=4, F=256, Fs=128)
    x = synth.activations(96, 32, 512)
    W = gu.upload(L)
    y1, r1 = gu.run_forward(W, gu.x_to_device(x=x))
    y2, r2 = gu.run_forward(W, gu.x_to_device(x=x))
    assert torch.equal(y1, y2) and torch.equal(r1.perm, r2.perm) and torch.equal(r1.topk_w, r2.topk_w)
    # a row gives the same result inside another batch on the same (batched)
    # path: its activation codes and products do not depend on the other rows
    ys, rs = gu.run_forward(W, gu.x_to_device(x=x[5:26]))
    for t in (5, 7, 25):
        assert torch.equal(rs.topk_idx[t - 5], r1.topk_idx[t])
        gu.assert_close(ys.cpu().numpy()[t - 5], y1.cpu().numpy()[t], tol=1e-5)
    # and alone, on the one-token schedule (other kernels and activation
    # coding), within the fp32 bound
    for t in (0, 7, 31):
        yt, rt = gu.run_forward(W, gu.x_to_device(x=x[t:t + 1]))
        assert torch.equal(rt.topk_idx[0], r1.topk_idx[t])
        gu.assert_close(yt.cpu().numpy()[0], y1.cpu().numpy()[t])


def test_route_then_expert_ffn_matches_layer_forward():
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(97, 0, D=512, E=32, k=4, F=256, Fs=128)
    x = gu.x_to_device(x=synth.activations(98, 11, 512))
    W = gu.upload(L)
    ws = moe.alloc_workspace(W, 11)
    r = moe.Routing(11, 4, 32)
    moe.route(W, x, r, ws)
    y = torch.zeros((11, 512), dtype=torch.float32, device="cuda")
    moe.expert_ffn(W, x, r, y, ws)
    y2, _ = gu.run_forward(W, x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("T", [1, 3, 40])
def test_stages_equal_layer_forward(T):
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(103, 0, D=512, E=32, k=4, F=256, Fs=128)
    x = gu.x_to_device(x=synth.activations(104, T, 512))
    W = gu.upload(L)
    ws = moe.alloc_workspace(W, T)
    r = moe.Routing(T, 4, 32)
    y = torch.zeros((T, 512), dtype=torch.float32, device="cuda")
    for st in (1, 2, 3, 4):
        moe.layer_forward_stage(W, x, y, ws, st, routing=r)
    y2, r2 = gu.run_forward(W, x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(r.perm, r2.perm)


@pytest.mark.parametrize("T,bf16", [(3, False), (40, False), (40, True)])
def test_stage5_repeats_the_routed_gate_up(T, bf16):
    # stage 5 runs the routed gate/up kernel alone on what stage 3 left in the
    # workspace (the grouped GEMM's activation codes and tiles; elsewhere it is
    # stage 3): stages 1, 2, 3, 5, 4 give the same y as one forward call
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(105, 0, D=512, E=32, k=4, F=256, Fs=128)
    xv = synth.activations(106, T, 512)
    x = gu.x_to_device(x_bf16=synth.to_bf16_bits(xv)) if bf16 else gu.x_to_device(x=xv)
    W = gu.upload(L)
    mode = moe.BF16 if bf16 else moe.F32
    ws = moe.alloc_workspace(W, T, mode)
    r = moe.Routing(T, 4, 32)
    y = torch.zeros((T, 512), dtype=torch.float32, device="cuda")
    for st in (1, 2, 3, 5, 4):
        moe.layer_forward_stage(W, x, y, ws, st, routing=r)
    y2, _ = gu.run_forward(W, x)
    torch.cuda.synchronize()
    if bf16:  # the routed down adds into y with atomics in a varying order
        gu.assert_close(y.cpu().numpy(), y2.cpu().numpy(), tol=1e-5)
    else:
        assert torch.equal(y, y2)


@pytest.mark.parametrize("D", [4096, 1000])
def test_rmsnorm(D):
    # 4096: the vector kernel (16-byte loads held in registers); 1000: the
    # general one
    import quantized_routed_moe_router_amd as moe
    x = synth.activations(99, 8, D)
    g = (0.9 + 0.2 * synth.uniform(99, 0, synth.TAG_GAMMA, 0, D)).astype(np.float32)
    ref = oracle.rmsnorm(x, g, 1e-6)
    xd, gd = gu.dev(x), gu.dev(g)
    out = torch.empty_like(xd)
    moe.rmsnorm(xd, gd, out, 1e-6)
    moe.rmsnorm(xd, gd, xd, 1e-6)  # in place
    torch.cuda.synchronize()
    gu.assert_close(out.cpu().numpy(), ref, tol=1e-5)
    assert torch.equal(out, xd)


def test_graph_replays_match_eager():
    # the block captured into a HIP graph, replayed several times with eager
    # work and synchronizations between replays; every replay must equal the
    # eager result bit for bit
    import quantized_routed_moe_router_amd as moe
    L = synth.make_layer(100, 0, D=512, E=32, k=4, F=256, Fs=128)
    W = gu.upload(L)
    xa = gu.x_to_device(x=synth.activations(101, 3, 512))
    xb = gu.x_to_device(x=synth.activations(102, 3, 512))
    ws = moe.alloc_workspace(W, 3)
    r = moe.Routing(3, 4, 32)
    y = torch.zeros((3, 512), dtype=torch.float32, device="cuda")
    moe.layer_forward(W, xa, y, ws, routing=r)
    torch.cuda.synchronize()
    eager = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            moe.layer_forward(W, xa, y, ws, routing=r)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), "replay %d" % rep
        yb = torch.zeros_like(y)
        moe.layer_forward(W, xb, yb, ws)  # other eager work on the same workspace
        torch.cuda.synchronize()


def test_bf16_shared_expert_beside_the_routed_path():
    # bf16 rows on the matrix-core path run the shared expert on a second
    # stream that the routed down waits for: eager (the layer, and route then
    # expert_ffn, both plain and accumulating into y) and the layer captured
    # into a HIP graph, whose fork and join are captured too, replayed with
    # eager work between the replays, all against the oracle
    import quantized_routed_moe_router_amd as moe
    T = 40
    L = synth.make_layer(110, 0, D=512, E=16, k=4, F=512, Fs=256)
    x = synth.activations(111, T, 512)
    xb = synth.to_bf16_bits(x)
    y_ref, idx_ref, w_ref = oracle.moe_forward(L, x_bf16=xb)
    W = gu.upload(L)
    xd = gu.x_to_device(x_bf16=xb)
    ws = moe.alloc_workspace(W, T, moe.BF16)
    r = moe.Routing(T, 4, 16)
    y = torch.zeros((T, 512), dtype=torch.float32, device="cuda")
    moe.layer_forward(W, xd, y, ws, routing=r)
    torch.cuda.synchronize()
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)
    gu.assert_close(y.cpu().numpy(), y_ref)
    y2 = torch.full((T, 512), 0.25, dtype=torch.float32, device="cuda")
    moe.expert_ffn(W, xd, r, y2, ws, accumulate=True)
    y3 = torch.zeros_like(y2)
    moe.expert_ffn(W, xd, r, y3, ws)
    torch.cuda.synchronize()
    gu.assert_close(y2.cpu().numpy(), y_ref + np.float32(0.25))
    gu.assert_close(y3.cpu().numpy(), y_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            moe.layer_forward(W, xd, y, ws, routing=r)
    torch.cuda.current_stream().wait_stream(side)
    xo = gu.x_to_device(x_bf16=synth.to_bf16_bits(synth.activations(112, T, 512)))
    for rep in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        gu.assert_close(y.cpu().numpy(), y_ref, what="y, replay %d" % rep)
        yo = torch.zeros_like(y)
        moe.layer_forward(W, xo, yo, ws)  # other eager work on the same workspace
        torch.cuda.synchronize()


def test_selection_counts_and_hotlist_bit_exact():
    # counts per {layer, expert} merged over 43 layers of routings (one from a
    # real forward, with out-of-range entries mixed in elsewhere), then hot
    # lists with many ties, a size that is not a power of two, one entry, the
    # largest size and counts beyond the sort key's range
    import quantized_routed_moe_router_amd as moe
    rng = np.random.default_rng(11)
    E, n_layer = 256, 43
    counts = torch.zeros(n_layer * E, dtype=torch.int64, device="cuda")
    ref = np.zeros(n_layer * E, np.int64)
    L = synth.make_layer(105, 0, D=256, E=E, k=6, F=128, Fs=0)
    W = gu.upload(L)
    y, r = gu.run_forward(W, gu.x_to_device(x=synth.activations(106, 9, 256)))
    for layer in range(n_layer):
        if layer == 0:
            idx = r.topk_idx.cpu().numpy()
        else:
            T = int(rng.integers(1, 40))
            idx = rng.integers(-2, E + 2, size=(T, 6)).astype(np.int32)
        moe.count_selections(gu.dev(idx), E, layer, counts)
        oracle.count_selections(idx, E, layer, ref)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), ref)
    cases = [ref, rng.integers(0, 5, size=11008), rng.integers(0, 3, size=16384), np.array([7]),
             np.array([0, 0, 0]), np.array([2 ** 40, 2 ** 39 - 1, 2 ** 39, 5, -3, 5])]
    for c in cases:
        c = np.asarray(c, np.int64)
        order = torch.empty(c.size, dtype=torch.int32, device="cuda")
        n_hot = torch.empty(1, dtype=torch.int32, device="cuda")
        moe.hotlist(gu.dev(c), order, n_hot)
        o_ref, nh_ref = oracle.hotlist(c)
        torch.cuda.synchronize()
        assert np.array_equal(order.cpu().numpy(), o_ref), c.size
        assert int(n_hot.item()) == nh_ref
