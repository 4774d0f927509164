"""GPU parity at the full workload sizes (n_embd 4096, 256 experts, top-6,
FFN width 2048, Q8_0 shared expert), in the launch configuration the
benchmark times.  Routing is compared for every row; outputs on sampled rows
the oracle computes one by one."""
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


def _run(wl, W, rows):
    kw = dict(x_bf16=wl.x_bf16) if wl.x_bf16 is not None else dict(x=wl.x)
    L = wl.layers[0]
    t = time.time()
    lg = oracle.logits(L, **kw)
    idx_ref, w_ref, gap = oracle.topk(lg, L.n_expert_used, L.route_scale)
    y_ref, _, _ = oracle.moe_forward(L, rows=rows, **kw)
    _log("%s: oracle %.1f s, min top-k margin %.3g" % (wl.name, time.time() - t, gap.min()))
    y, r = gu.run_forward(W if L.router_bias is None else gu.upload_bias(W, L), gu.x_to_device(**kw))
    gu.check_routing(r, idx_ref, w_ref, L.n_expert)
    worst = gu.assert_close(y.cpu().numpy()[rows], y_ref[rows])
    _log("%s: worst relative error %.3g" % (wl.name, worst))


def test_decode_b1(flash):
    L, W = flash
    _run(synth.decode_b1(L), W, [0])


def test_decode_b32_zipf(flash):
    L, W = flash
    _run(synth.decode_b32(L), W, [0, 5, 17, 31])


def test_prefill_2048(flash):
    L, W = flash
    _run(synth.prefill_2048(L), W, [0, 1, 511, 1024, 2047])
