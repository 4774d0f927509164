"""Helpers shared by the GPU tests: upload a synth.Layer, run the library,
compare with the oracle at the stated tolerance, and compute the oracle's
output of many rows on the host cores."""
import concurrent.futures
import os

import numpy as np
import torch

import quantized_routed_moe_router_amd as moe

TOL = 2e-3  # |gpu - ref| <= TOL * (1 + |ref|) on fp32 outputs


def dev(a):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def upload(L):
    return moe.LayerWeights(
        n_embd=L.n_embd, n_expert=L.n_expert, n_expert_used=L.n_expert_used, n_ff_exp=L.n_ff_exp,
        n_ff_shared=L.n_ff_shared, gate_type=L.gate_fmt, up_type=L.up_fmt, down_type=L.down_fmt,
        shared_type=L.shared_fmt, router_w=dev(L.router_w), gate=dev(L.gate), up=dev(L.up), down=dev(L.down),
        sh_gate=dev(L.sh_gate), sh_up=dev(L.sh_up), sh_down=dev(L.sh_down), router_bias=dev(L.router_bias),
        route_scale=L.route_scale, codebook=dev(L.codebook), gamma=dev(L.gamma))


def x_to_device(x=None, x_bf16=None):
    if x_bf16 is not None:
        return torch.from_numpy(np.ascontiguousarray(x_bf16).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def run_forward(W, xd, accumulate=False, y0=None, routing=True):
    T = xd.shape[0]
    ws = moe.alloc_workspace(W, T, moe.BF16 if xd.dtype == torch.bfloat16 else moe.F32)
    y = y0.clone() if y0 is not None else torch.zeros((T, W.n_embd), dtype=torch.float32, device="cuda")
    r = moe.Routing(T, W.n_expert_used, W.n_expert) if routing else None
    moe.layer_forward(W, xd, y, ws, routing=r, accumulate=accumulate)
    torch.cuda.synchronize()
    return y, r


def assert_close(got, ref, tol=TOL, what="y"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = tol * (1.0 + np.abs(ref))
    bad = err > bound
    assert not bad.any(), "%s: %d of %d elements out of tolerance; worst |err|=%.3g at ref=%.3g" % (
        what, int(bad.sum()), bad.size, err.max(), ref.flat[int(np.argmax(err / bound))])
    return float((err / (1.0 + np.abs(ref))).max())


def check_routing(r, idx_ref, w_ref, E):
    import oracle
    idx = r.topk_idx.cpu().numpy()
    assert np.array_equal(idx, idx_ref), "topk_idx differs in %d places" % int((idx != idx_ref).sum())
    assert_close(r.topk_w.cpu().numpy(), w_ref, what="topk_w")
    b = oracle.bucket(idx_ref, E)
    for name in ("count", "offset", "perm", "pos", "n_active"):
        got = getattr(r, name).cpu().numpy()
        assert np.array_equal(got, b[name]), name
    na = int(b["n_active"][0])
    act = r.active.cpu().numpy()
    assert np.array_equal(act[:na], b["active"][:na]) and np.all(act[na:] == -1)


def upload_bias(W, L):
    """Same device weights with the layer's router bias attached."""
    import copy
    W2 = copy.copy(W)
    W2.router_bias = dev(L.router_bias)
    return W2


def oracle_workers():
    """Host threads for the oracle fan-out (at most 16, the CPU share of one GPU)."""
    return max(1, min(16, os.cpu_count() or 1))


def oracle_all_rows(L, x=None, x_bf16=None, workers=None):
    """(y [T][D], topk_idx, topk_w) of every row from the oracle, with the rows
    cut into chunks evaluated on a thread pool.  The oracle's C call releases
    the interpreter lock, and a row's result does not depend on the other
    rows of its call (batching is exact), so the chunks equal one call over
    all rows."""
    import oracle
    src = x_bf16 if x_bf16 is not None else x
    T = src.shape[0]
    n = workers or oracle_workers()
    # several chunks per worker so that an uneven chunk does not hold the pool
    step = max(1, -(-T // (4 * n)))
    cuts = [(a, min(T, a + step)) for a in range(0, T, step)]

    def one(ab):
        a, b = ab
        kw = dict(x_bf16=x_bf16[a:b]) if x_bf16 is not None else dict(x=x[a:b])
        return oracle.moe_forward(L, **kw)

    with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
        parts = list(ex.map(one, cuts))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
            np.concatenate([p[2] for p in parts]))


def oracle_stack(layers, x, teacher=None, workers=None):
    """oracle.stack_forward with the rows evaluated one by one on a thread pool
    (every step of a block is row by row, so the rows are independent)."""
    import oracle
    T = x.shape[0]
    n = workers or oracle_workers()

    def one(t):
        tf = None if teacher is None else [tt[t:t + 1] for tt in teacher]
        return oracle.stack_forward(layers, x[t:t + 1], teacher=tf)

    with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
        parts = list(ex.map(one, range(T)))
    return [np.concatenate([p[l] for p in parts]) for l in range(len(layers))]
