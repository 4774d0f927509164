"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: figures the
pages print, hand-built blocks with hand-computed values, brute force on tiny
inputs, closed forms, textbook numpy float64 algebra, and round trips through
the independent generator's encoders.  No GPU.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        return json.load(f)


# ---- shapes and byte counts (pages' printed figures) ---------------------------

def test_params_match_pages():
    pg = _page()
    s = pg["flash_shape"]
    D, F, E, k, nl = s["n_embd"], s["n_ff_exp"], s["n_expert"], s["n_expert_used"], s["n_layer"]
    per_expert = 3 * D * F
    assert per_expert == 25_165_824
    assert round(per_expert / 1e6, 1) == pg["params"]["per_expert_millions_approx"]
    assert round(per_expert * E / 1e9, 2) == pg["params"]["per_layer_billions_approx"]
    assert round(per_expert * E * nl / 1e9) == pg["params"]["routed_billions_approx"]
    assert round(100 * k / E, 2) == pg["params"]["active_percent_approx"]
    assert round(100 * 277 / pg["params"]["total_billions"], 1) == pg["params"]["routed_share_percent_approx"]
    assert round(100 * (E - k) / E, 1) == pg["skipped_ffn_percent"]["value"]
    # the workload recipe carries the same shape
    assert synth.DS4_FLASH == dict(D=D, E=E, k=k, F=F, Fs=F, n_layer=nl)


def test_block_sizes_match_pages():
    pg = _page()["block_sizes"]
    assert oracle.tensor_bytes(oracle.Q2K, 256) == pg["q2k_bytes"]
    assert oracle.tensor_bytes(oracle.CB2, 256) == pg["cb2_bytes"]
    assert 8 * pg["q2k_bytes"] / 256 == pg["q2k_bits"]
    assert 8 * pg["cb2_bytes"] / 256 == pg["cb2_bits"]
    assert oracle.tensor_bytes(oracle.Q8_0, 32) == 34  # 32 int8 + fp16 scale
    assert oracle.tensor_bytes(oracle.Q2K, 255) == -1  # partial blocks rejected


def test_stack_routed_bytes_match_pages():
    pg = _page()
    s = pg["flash_shape"]
    D, F, E, nl = s["n_embd"], s["n_ff_exp"], s["n_expert"], s["n_layer"]
    per_expert = 2 * oracle.tensor_bytes(oracle.CB2, F * D) + oracle.tensor_bytes(oracle.Q2K, D * F)
    assert per_expert == 7_077_888
    total = per_expert * E * nl
    bpw = 8 * total / (3 * D * F * E * nl)
    # the pages: 277B at ~2.23 bits ~ 77 GB; gate/up at 2.0625 and down at 2.625 bits give 2.25
    assert abs(bpw - pg["routed_size"]["bits_per_weight_approx"]) < 0.03
    assert abs(total / 1e9 - pg["routed_size"]["gb_approx"]) < 0.03 * pg["routed_size"]["gb_approx"]


# ---- dequantization closed forms (hand-built blocks) --------------------------

def _q2k_block(d_bits, dmin_bits, sc, mn, q):
    b = np.zeros(84, np.uint8)
    b[0:2] = np.frombuffer(np.uint16(d_bits).tobytes(), np.uint8)
    b[2:4] = np.frombuffer(np.uint16(dmin_bits).tobytes(), np.uint8)
    for g in range(16):
        b[4 + g] = (sc[g] & 15) | ((mn[g] & 15) << 4)
    for i in range(256):
        b[20 + i // 4] |= (q[i] & 3) << (2 * (i % 4))
    return b


F16_ONE, F16_HALF, F16_QUARTER = 0x3C00, 0x3800, 0x3400


def test_q2k_closed_forms():
    z = oracle.dequant(oracle.Q2K, np.zeros(84, np.uint8), 256)
    assert np.all(z == 0) and not np.any(np.signbit(z))
    w = oracle.dequant(oracle.Q2K, _q2k_block(F16_ONE, 0, [15] * 16, [0] * 16, [3] * 256), 256)
    assert np.all(w == 45.0)
    w = oracle.dequant(oracle.Q2K, _q2k_block(F16_ONE, F16_ONE, [1] * 16, [1] * 16, [0] * 256), 256)
    assert np.all(w == -1.0)
    # d = 0.5, dmin = 0.25, group g has scale g and min 15-g, code i % 4
    sc = list(range(16))
    mn = [15 - g for g in range(16)]
    w = oracle.dequant(oracle.Q2K, _q2k_block(F16_HALF, F16_QUARTER, sc, mn, [i % 4 for i in range(256)]), 256)
    assert w[49] == -1.5      # group 3: 0.5*3*1 - 0.25*12
    assert w[255] == 22.5     # group 15: 0.5*15*3 - 0
    assert w[0] == -3.75      # group 0: 0 - 0.25*15
    assert w[130] == 6.25  # group 8: 0.5*8*2 - 0.25*7
    # a group takes at most 4 values spaced d*scale apart
    for g in range(16):
        vals = np.unique(w[16 * g:16 * g + 16])
        assert len(vals) <= 4
        if len(vals) > 1:
            assert np.allclose(np.diff(vals), 0.5 * sc[g])


def test_q2k_bit_positions():
    for i in (0, 5, 15, 16, 77, 255):
        q = [0] * 256
        q[i] = 1
        w = oracle.dequant(oracle.Q2K, _q2k_block(F16_ONE, 0, [1] * 16, [0] * 16, q), 256)
        expect = np.zeros(256, np.float32)
        expect[i] = 1.0
        assert np.array_equal(w, expect), i
    # scale nibble of group 9 only
    sc = [0] * 16
    sc[9] = 7
    w = oracle.dequant(oracle.Q2K, _q2k_block(F16_ONE, 0, sc, [0] * 16, [2] * 256), 256)
    assert np.all(w[144:160] == 14.0) and np.count_nonzero(w) == 16


def test_q2k_subnormal_scale():
    w = oracle.dequant(oracle.Q2K, _q2k_block(0x0001, 0, [1] * 16, [0] * 16, [1] * 256), 256)
    assert np.all(w == np.float32(2.0 ** -24))


def _q4k_block(d_bits, dmin_bits, sc, mn, q):
    # written from the header's layout, apart from both encoders and decoders
    b = np.zeros(144, np.uint8)
    b[0:2] = np.frombuffer(np.uint16(d_bits).tobytes(), np.uint8)
    b[2:4] = np.frombuffer(np.uint16(dmin_bits).tobytes(), np.uint8)
    bits = 0
    for f, v in enumerate(list(sc) + list(mn)):
        bits |= (int(v) & 63) << (6 * f)
    b[4:16] = np.frombuffer(bits.to_bytes(12, "little"), np.uint8)
    for i in range(256):
        b[16 + i // 2] |= (q[i] & 15) << (4 * (i % 2))
    return b


def test_q4k_closed_forms():
    # "Understanding Dwarf Star" 2.3.2, the Q4_K layout: w = d*scale_j*q - dmin*min_j
    z = oracle.dequant(oracle.Q4K, np.zeros(144, np.uint8), 256)
    assert np.all(z == 0) and not np.any(np.signbit(z))
    w = oracle.dequant(oracle.Q4K, _q4k_block(F16_ONE, 0, [63] * 8, [0] * 8, [15] * 256), 256)
    assert np.all(w == 945.0)
    w = oracle.dequant(oracle.Q4K, _q4k_block(F16_ONE, F16_ONE, [1] * 8, [1] * 8, [0] * 256), 256)
    assert np.all(w == -1.0)
    # d = 0.5, dmin = 0.25, sub-block j has scale 8j+1 and min 63-8j, code i % 16
    sc = [8 * j + 1 for j in range(8)]
    mn = [63 - 8 * j for j in range(8)]
    w = oracle.dequant(oracle.Q4K, _q4k_block(F16_HALF, F16_QUARTER, sc, mn, [i % 16 for i in range(256)]), 256)
    assert w[37] == 0.5 * 9 * 5 - 0.25 * 55     # sub-block 1, code 5
    assert w[255] == 0.5 * 57 * 15 - 0.25 * 7   # sub-block 7, code 15


def test_q4k_bit_positions():
    for i in (0, 1, 30, 31, 32, 129, 255):
        q = [0] * 256
        q[i] = 9
        w = oracle.dequant(oracle.Q4K, _q4k_block(F16_ONE, 0, [1] * 8, [0] * 8, q), 256)
        expect = np.zeros(256, np.float32)
        expect[i] = 9.0
        assert np.array_equal(w, expect), i
    # each 6-bit field reaches exactly its own sub-block, as scale or as min
    for f in range(16):
        sc, mn = [0] * 8, [0] * 8
        (sc if f < 8 else mn)[f % 8] = 37
        w = oracle.dequant(oracle.Q4K, _q4k_block(F16_ONE, F16_ONE, sc, mn, [2] * 256), 256)
        j = f % 8
        expect = np.zeros(256, np.float32)
        expect[32 * j:32 * j + 32] = 74.0 if f < 8 else -37.0
        assert np.array_equal(w, expect), f


def test_q8_0_closed_form():
    b = np.zeros(34, np.uint8)
    b[0:2] = np.frombuffer(np.uint16(F16_HALF).tobytes(), np.uint8)
    q = np.array([-127, -1, 0, 1, 127] + [3] * 27, np.int8)
    b[2:] = q.view(np.uint8)
    w = oracle.dequant(oracle.Q8_0, b, 32)
    assert list(w[:5]) == [-63.5, -0.5, 0.0, 0.5, 63.5] and np.all(w[5:] == 1.5)


def test_cb2_closed_form():
    cb = np.zeros((256, 8), np.int8)
    cb[7] = [1, -2, 3, -4, 5, -6, 7, -8]
    cb[200] = [8, 8, 0, 0, -8, -8, 1, -1]
    b = np.zeros(66, np.uint8)
    b[0:2] = np.frombuffer(np.uint16(0x4000).tobytes(), np.uint8)  # d = 2
    b[2] = 7
    b[34] = 0b00000101  # flip weights 0 and 2
    b[2 + 31] = 200
    b[34 + 31] = 0b10000000
    w = oracle.dequant(oracle.CB2, b, 256, codebook=cb)
    assert list(w[:8]) == [-2, -4, -6, -8, 10, -12, 14, -16]
    assert list(w[248:]) == [16, 16, 0, 0, -16, -16, 2, 2]
    assert np.all(w[8:248] == 0)


def test_dequant_round_trips_through_encoders():
    # the generator's encoders and the oracle's decoders are written apart;
    # a wrong byte or bit order in either breaks these bounds
    n = 64 * 256
    v = synth.normal(11, 0, 99, 0, n, 0.02)
    for fmt in (synth.Q2K, synth.Q8_0, synth.Q4K):
        b = synth.expert_tensor(fmt, 11, 0, 99, 1, n // 256, 256)
        w = oracle.dequant(fmt, b, n)
        err = np.abs(w - v)
        if fmt == synth.Q8_0:
            d = np.abs(v).reshape(-1, 32).max(1) / 127
            assert np.all(err.reshape(-1, 32) <= 0.5001 * d[:, None] + 1e-7)
        elif fmt == synth.Q4K:  # sub-blocks of 32, codes 0..15
            blk = v.reshape(-1, 8, 32)
            rng = blk.max(2) - np.minimum(blk.min(2), 0)
            step = rng / 15
            assert np.all(err.reshape(-1, 8, 32) <= 0.75 * step.max(1)[:, None, None] + 1e-4)
            assert err.mean() < 0.1 * 0.02  # 4-bit codes: a small fraction of sigma
        else:
            blk = v.reshape(-1, 16, 16)
            rng = blk.max(2) - np.minimum(blk.min(2), 0)
            step = rng / 3
            assert np.all(err.reshape(-1, 16, 16) <= 0.75 * step.max(1)[:, None, None] + 1e-4)
            assert err.mean() < 0.35 * 0.02  # 2-bit codes: about a quarter of a step on average
    cb = synth.codebook(4)
    b = synth.expert_tensor(synth.CB2, 11, 0, 99, 1, n // 256, 256, codebook=cb)
    w = oracle.dequant(oracle.CB2, b, n, codebook=cb)
    nz = w != 0
    assert np.all(np.sign(w[nz]) == np.sign(v[nz]))
    d = np.array([oracle.dequant(oracle.Q8_0, np.concatenate([b[66 * i:66 * i + 2], np.ones(32, np.uint8)]), 32)[0]
                  for i in range(n // 256)])
    mags = np.abs(w).reshape(-1, 256) / d[:, None]
    idx = b.reshape(-1, 66)[:, 2:34]
    assert np.array_equal(mags, np.abs(cb[idx].reshape(-1, 256).astype(np.float32)))


# ---- routing -----------------------------------------------------------------

def _brute_topk(l, k):
    E = len(l)
    best = None
    for S in itertools.combinations(range(E), k):
        out = [e for e in range(E) if e not in S]
        ok = all(l[a] > l[b] or (l[a] == l[b] and a < b) for a in S for b in out)
        if ok:
            assert best is None
            best = S
    return sorted(best, key=lambda e: (-l[e], e))


def test_topk_brute_force():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((60, 8))
    lg[::7, 3] = lg[::7, 5]            # exact ties
    lg[::9, :] = 0.25                  # all equal
    idx, w, _ = oracle.topk(lg, 3)
    for t in range(lg.shape[0]):
        assert list(idx[t]) == _brute_topk(list(lg[t]), 3)
        p = softmax(lg[t])
        sel = p[idx[t]]
        assert np.allclose(w[t], sel / sel.sum(), rtol=1e-6, atol=0)


def test_topk_invariances():
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((40, 32)) * 2
    i1, w1, _ = oracle.topk(lg, 6)
    i2, w2, _ = oracle.topk(lg + 3.0, 6)
    assert np.array_equal(i1, i2) and np.allclose(w1, w2, rtol=1e-6)
    assert np.allclose(w1.sum(1), 1.0, atol=1e-6)
    i3, w3, _ = oracle.topk(lg, 6, route_scale=1.5)
    assert np.array_equal(i1, i3) and np.allclose(w3, 1.5 * w1, rtol=1e-6)
    assert np.all(np.diff(lg[np.arange(40)[:, None], i1], axis=1) <= 0)
    # with k = E the weights are the full softmax
    i4, w4, gap = oracle.topk(lg[:, :6], 6)
    full = softmax(lg[:, :6], axis=1)
    assert np.allclose(np.take_along_axis(full, i4, 1), w4, rtol=1e-6)
    assert np.all(np.isinf(gap))


def test_router_logits_and_duplicate_columns():
    L = synth.make_layer(21, 0, D=256, E=16, k=2, F=128, Fs=0)
    x = synth.activations(21, 9, 256)
    lg = oracle.logits(L, x=x)
    ref = x.astype(np.float64) @ L.router_w.astype(np.float64).T
    assert np.allclose(lg, ref, rtol=1e-12, atol=1e-12)
    # duplicated router rows tie exactly; the lower index is taken first
    W = L.router_w.copy()
    W[11] = W[4]
    L.router_w = W
    bias = np.zeros(16, np.float32)
    bias[4] = bias[11] = 50.0
    L.router_bias = bias
    idx, w, gap = oracle.route(L, x=x)
    assert np.all(idx[:, 0] == 4) and np.all(idx[:, 1] == 11)
    assert np.all(w[:, 0] == w[:, 1])


def test_bucket_matches_stable_sort():
    rng = np.random.default_rng(7)
    for T, k, E in ((1, 6, 256), (32, 6, 256), (513, 2, 16), (7, 3, 5)):
        idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32)
        b = oracle.bucket(idx, E)
        flat = idx.reshape(-1)
        assert np.array_equal(b["count"], np.bincount(flat, minlength=E))
        assert b["offset"][0] == 0 and np.array_equal(np.diff(b["offset"]), b["count"])
        assert np.array_equal(b["perm"], np.argsort(flat, kind="stable"))
        assert np.array_equal(b["pos"][b["perm"]], np.arange(T * k))
        act = np.nonzero(b["count"])[0]
        assert b["n_active"][0] == len(act) and np.array_equal(b["active"][:len(act)], act)


# ---- the FFN and the block -----------------------------------------------------

def _silu(z):
    return z / (1.0 + np.exp(-z))


def _round_bf16(a):
    f = np.asarray(a, np.float32).copy()
    u = f.view(np.uint32)
    u[:] = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return f.astype(np.float64)


def _dense_numpy(L, xd, bf16=False):
    D, F, E = L.n_embd, L.n_ff_exp, L.n_expert
    nb = lambda fmt, n: synth.tensor_bytes(fmt, n)

    def mat(buf, fmt, e, rows, cols):
        sz = nb(fmt, rows * cols)
        return oracle.dequant(fmt, buf[e * sz:(e + 1) * sz], rows * cols, L.codebook).astype(np.float64).reshape(rows, cols)

    def ffn(g, u, d, x):
        h = _silu(x @ g.T) * (x @ u.T)
        if bf16:
            h = _round_bf16(h)
        return h @ d.T

    y = np.zeros((xd.shape[0], D))
    if L.n_ff_shared:
        Fs = L.n_ff_shared
        y += ffn(mat(L.sh_gate, L.shared_fmt, 0, Fs, D), mat(L.sh_up, L.shared_fmt, 0, Fs, D),
                 mat(L.sh_down, L.shared_fmt, 0, D, Fs), xd)
    lg = xd @ L.router_w.astype(np.float64).T
    if L.router_bias is not None:
        lg = lg + L.router_bias.astype(np.float64)
    for t in range(xd.shape[0]):
        sel = sorted(range(E), key=lambda e: (-lg[t, e], e))[:L.n_expert_used]
        p = np.exp(lg[t, sel] - lg[t, sel].max())
        p = L.route_scale * p / p.sum()
        for e, pe in zip(sel, p):
            y[t] += pe * ffn(mat(L.gate, L.gate_fmt, e, F, D), mat(L.up, L.up_fmt, e, F, D),
                             mat(L.down, L.down_fmt, e, D, F), xd[t:t + 1])[0]
    return y


@pytest.mark.parametrize("shared", [False, True])
def test_single_expert_is_a_dense_swiglu(shared):
    L = synth.make_layer(31, 0, D=256, E=1, k=1, F=128, Fs=64 if shared else 0)
    x = synth.activations(31, 5, 256)
    y, idx, w = oracle.moe_forward(L, x=x)
    assert np.all(idx == 0) and np.all(w == 1.0)
    ref = _dense_numpy(L, x.astype(np.float64))
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-7)


def test_block_matches_numpy_definition():
    L = synth.make_layer(32, 0, D=256, E=8, k=3, F=128, Fs=64)
    L.route_scale = 1.5
    x = synth.activations(32, 6, 256)
    y, _, _ = oracle.moe_forward(L, x=x)
    assert np.allclose(y, _dense_numpy(L, x.astype(np.float64)), rtol=1e-6, atol=1e-7)
    # gate and up are not interchangeable (silu sits on the gate)
    L2 = synth.make_layer(32, 0, D=256, E=8, k=3, F=128, Fs=64)
    L2.gate, L2.up = L2.up, L2.gate
    y2, _, _ = oracle.moe_forward(L2, x=x)
    assert not np.allclose(y2, y, atol=1e-3)


def test_bf16_mode_matches_numpy_definition():
    # the bf16 workload casts the activations to bf16 and nothing else: the
    # block on bf16 x is the numpy definition on x's bf16 values, and it is
    # bit for bit the fp32 mode on those same values (bf16 -> fp32 is exact)
    L = synth.make_layer(33, 0, D=256, E=8, k=2, F=128, Fs=64)
    xb = synth.to_bf16_bits(synth.activations(33, 5, 256))
    y, idx, w = oracle.moe_forward(L, x_bf16=xb)
    xd = oracle.input_as_double(x_bf16=xb)
    assert np.allclose(y, _dense_numpy(L, xd), rtol=1e-6, atol=1e-7)
    y32, idx32, w32 = oracle.moe_forward(L, x=xd.astype(np.float32))
    assert np.array_equal(y, y32) and np.array_equal(idx, idx32) and np.array_equal(w, w32)
    # rounding h to bf16 as well would move the result
    assert not np.allclose(y, _dense_numpy(L, xd, bf16=True), rtol=1e-7, atol=0)


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_sparse_equals_dense_exactly(mode):
    wl = synth.tiny()
    L = wl.layers[0]
    kw = dict(x=wl.x) if mode == "f32" else dict(x_bf16=synth.to_bf16_bits(wl.x))
    y, _, _ = oracle.moe_forward(L, **kw)
    yd = oracle.moe_forward_dense(L, **kw)
    assert np.array_equal(y, yd)
    L2 = synth.make_layer(34, 0, D=256, E=12, k=4, F=64, Fs=128)
    x2 = synth.activations(34, 3, 256)
    kw2 = dict(x=x2) if mode == "f32" else dict(x_bf16=synth.to_bf16_bits(x2))
    assert np.array_equal(oracle.moe_forward(L2, **kw2)[0], oracle.moe_forward_dense(L2, **kw2))


def test_zero_gate_or_up_gives_zero():
    L = synth.make_layer(35, 0, D=256, E=4, k=2, F=64, Fs=0)
    x = synth.activations(35, 3, 256)
    Lz = synth.make_layer(35, 0, D=256, E=4, k=2, F=64, Fs=0)
    Lz.gate = np.zeros_like(L.gate)  # silu(0) = 0
    assert np.all(oracle.moe_forward(Lz, x=x)[0] == 0)
    Lz = synth.make_layer(35, 0, D=256, E=4, k=2, F=64, Fs=0)
    Lz.up = np.zeros_like(L.up)
    assert np.all(oracle.moe_forward(Lz, x=x)[0] == 0)


def test_batching_is_exact():
    # each row of a batch equals the same row evaluated alone
    L = synth.make_layer(36, 0, D=256, E=16, k=4, F=128, Fs=64)
    x = synth.activations(36, 7, 256)
    yb, ib, wb = oracle.moe_forward(L, x=x)
    for t in range(7):
        y1, i1, w1 = oracle.moe_forward(L, x=x[t:t + 1])
        assert np.array_equal(y1[0], yb[t]) and np.array_equal(i1[0], ib[t]) and np.array_equal(w1[0], wb[t])


def test_rows_subset_matches_full():
    L = synth.make_layer(37, 0, D=256, E=16, k=2, F=128, Fs=0)
    x = synth.activations(37, 6, 256)
    yf, _, _ = oracle.moe_forward(L, x=x)
    ys, _, _ = oracle.moe_forward(L, x=x, rows=[4, 1])
    assert np.array_equal(ys[[1, 4]], yf[[1, 4]]) and np.all(np.isnan(ys[[0, 2, 3, 5]]))


def test_rmsnorm_closed_form():
    D = 64
    g = np.linspace(0.9, 1.1, D).astype(np.float32)
    for c in (0.0, 1e-3, 1.0, -3.5):
        x = np.full((1, D), c, np.float32)
        out = oracle.rmsnorm(x, g, 1e-6)
        ref = g.astype(np.float64) * c / math.sqrt(c * c + 1e-6)
        assert np.allclose(out[0], ref, rtol=1e-7, atol=0)
    x = synth.activations(38, 3, D)
    ref = g * x / np.sqrt((x.astype(np.float64) ** 2).mean(1, keepdims=True) + 1e-6)
    assert np.allclose(oracle.rmsnorm(x, g), ref, rtol=1e-6)


def _stack_numpy(layers, x, eps=1e-6):
    """The stack written out in numpy float64 ("Understanding Dwarf Star" 5.2.1
    and 5.6.2: each block normalizes its input, and the block's output is added
    back to the un-normalized input): the normalized row is held in fp32 (the
    block's input type), the block is the numpy dense definition above, and its
    fp32 output is added to x in fp32."""
    outs, cur = [], np.asarray(x, np.float32)
    for L in layers:
        xd = cur.astype(np.float64)
        inv = 1.0 / np.sqrt(np.mean(xd * xd, axis=1, keepdims=True) + eps)
        xn = (L.gamma.astype(np.float64) * xd * inv).astype(np.float32)
        y = _dense_numpy(L, xn.astype(np.float64)).astype(np.float32)
        cur = cur + y
        outs.append(cur)
    return outs


@pytest.mark.parametrize("E,k", [(1, 1), (6, 2)])
def test_stack_matches_numpy_composition(E, k):
    # E = k = 1 makes each block a dense SwiGLU (plus the shared expert);
    # E = 6, k = 2 routes.  At activations of 1e-3 the mean square equals
    # eps, so a misplaced eps moves the result by sqrt(2); at 1 the norm
    # scales each row by gamma, so a residual added to the normalized row
    # instead of x moves it by up to 10%.
    layers = [synth.make_layer(41, l, D=256, E=E, k=k, F=64, Fs=64, gamma=True) for l in range(3)]
    for scale in (1.0, 1e-3):
        x = (synth.activations(41, 3, 256) * scale).astype(np.float32)
        got = oracle.stack_forward(layers, x)
        ref = _stack_numpy(layers, x)
        assert len(got) == 3
        for a, b in zip(got, ref):
            assert a.dtype == np.float32
            # one fp32 ulp of the normalized row may differ (the sums run in
            # another order) and moves outputs that cancel to near zero
            assert np.allclose(a, b, rtol=1e-5, atol=1e-6 * np.abs(b).max())
    # the layers differ (their own gamma and weights): repeating layer 0
    # three times gives another result
    x = synth.activations(41, 3, 256)
    assert not np.allclose(oracle.stack_forward([layers[0]] * 3, x)[2], oracle.stack_forward(layers, x)[2],
                           rtol=1e-4)


def test_stack_with_zero_experts_passes_x_through():
    # zero gate rows give silu(0) * u = 0, so every block adds exact zeros and
    # each layer's output is its input, bit for bit
    layers = []
    for l in range(3):
        L = synth.make_layer(42, l, D=256, E=8, k=2, F=64, Fs=64, gamma=True)
        L.gate = np.zeros_like(L.gate)
        L.sh_gate = np.zeros_like(L.sh_gate)
        layers.append(L)
    x = synth.activations(42, 4, 256)
    for out in oracle.stack_forward(layers, x):
        assert np.array_equal(out, x)


def test_stack_teacher_forcing_is_consistent():
    cb = synth.codebook(4)
    layers = [synth.make_layer(40, l, D=256, E=8, k=2, F=64, Fs=64, gate_fmt=synth.CB2, down_fmt=synth.Q2K,
                               cb=cb, gamma=True) for l in range(3)]
    x = synth.activations(40, 2, 256)
    free = oracle.stack_forward(layers, x)
    forced = oracle.stack_forward(layers, x, teacher=[x] + free[:-1])
    for a, b in zip(free, forced):
        assert np.array_equal(a, b)


# Selection counts and the hot list ("The sparsity that pays for everything
# else in DwarfStar", "Some experts run far more often than others").

def test_count_selections_is_a_histogram_and_merges():
    rng = np.random.default_rng(5)
    E, n_layer = 40, 3
    counts = np.zeros(n_layer * E, np.int64)
    expect = np.zeros(n_layer * E, np.int64)
    for layer, T, k in ((0, 7, 3), (2, 5, 6), (0, 4, 2)):  # layer 0 twice: the second merges
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
        oracle.count_selections(idx, E, layer, counts)
        expect[layer * E:(layer + 1) * E] += np.bincount(idx.ravel(), minlength=E)
    assert np.array_equal(counts, expect)
    assert counts.sum() == 7 * 3 + 5 * 6 + 4 * 2 and counts[E:2 * E].sum() == 0
    # indices outside [0, E) are not counted
    c2 = np.zeros(E, np.int64)
    oracle.count_selections(np.array([[-1, 0, E, 3]], np.int32), E, 0, c2)
    assert c2.sum() == 2 and c2[0] == 1 and c2[3] == 1


def test_hotlist_orders_by_hits_then_index():
    # a hand case: ties (5 at 1 and 4; 0 at 0, 3, 5) keep the lower index first
    order, n_hot = oracle.hotlist(np.array([0, 5, 9, 0, 5, 0, 2], np.int64))
    assert order.tolist() == [2, 1, 4, 6, 0, 3, 5] and n_hot == 4
    rng = np.random.default_rng(6)
    c = rng.integers(0, 12, size=43 * 256).astype(np.int64)  # many ties
    order, n_hot = oracle.hotlist(c)
    assert order.tolist() == sorted(range(c.size), key=lambda i: (-int(c[i]), i))
    assert n_hot == int((c > 0).sum())


def test_oracle_is_thread_safe():
    # the GPU parity tests evaluate the oracle's rows on a pool of threads;
    # every thread must get what a serial call gives (the top-k sort keys are
    # per thread)
    import concurrent.futures
    rng = np.random.default_rng(9)
    lgs = [rng.normal(size=(64, 256)) for _ in range(16)]
    serial = [oracle.topk(lg, 6) for lg in lgs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        for _ in range(4):
            par = list(ex.map(lambda lg: oracle.topk(lg, 6), lgs))
            for a, b in zip(serial, par):
                assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
