"""Seeded synthetic inputs for the routed mixture-of-experts block.

This package draws every input the block is run on: activations, router
matrix, optional router bias, RMSNorm weights, the codebook, and the expert
weights encoded into their block formats.  It holds none of the block's own
arithmetic (no decoding, routing or products), so the GPU library's tests and
the CPU oracle can both consume its bytes without sharing any method code.

Workload recipes (shapes from "Understanding Dwarf Star" 2.4.3 and the
"Where the parameters actually are" section of "The sparsity that pays for
everything else in DwarfStar": n_embd 4096, 256 routed experts, 6 used,
one shared expert, expert FFN width 2048, 43 layers):

  tiny           T=4, D=256, E=16, k=2, F=128, no shared expert, Q2K experts
  decode_b1      T=1, D=4096, E=256, k=6, F=2048, Q2K experts, Q8_0 shared
  decode_b32     T=32 on the same layer, router logits biased by ln Zipf(1.1)
  prefill_2048   T=2048 on the same layer, activations given as bf16
  stack43        43 blocks x += MoE(RMSNorm(x)), CB2 gate/up, Q2K down, B=1, 8
"""
import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import build as _build

F32, BF16, Q2K, Q8_0, CB2, Q4K = 0, 1, 2, 3, 4, 5
BLOCK_WEIGHTS = {Q2K: 256, Q8_0: 32, CB2: 256, Q4K: 256}
BLOCK_BYTES = {Q2K: 84, Q8_0: 34, CB2: 66, Q4K: 144}

# stream tags (one key per (seed, layer, tag, expert))
TAG_X, TAG_ROUTER, TAG_GATE, TAG_UP, TAG_DOWN = 1, 2, 3, 4, 5
TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN, TAG_GAMMA, TAG_CODEBOOK, TAG_PERM = 6, 7, 8, 9, 10, 11

WEIGHT_SIGMA = 0.02  # std of N(0, 0.02) expert, shared and router weights

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.sy_gen_expert_tensor.restype = ctypes.c_int64
        lib.sy_gen_expert_tensor.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.sy_gen_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        lib.sy_gen_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.sy_gen_codebook.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p]
        lib.sy_f32_to_f16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.sy_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.sy_key.restype = ctypes.c_uint64
        lib.sy_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        _lib = lib
    return _lib


def default_threads():
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def tensor_bytes(fmt, n_weights):
    bw = BLOCK_WEIGHTS[fmt]
    assert n_weights % bw == 0, (fmt, n_weights)
    return n_weights // bw * BLOCK_BYTES[fmt]


def expert_tensor(fmt, seed, layer, tag, n_expert, n_rows, n_in, sigma=WEIGHT_SIGMA, codebook=None,
                  nthreads=None):
    """n_expert matrices [n_rows][n_in] of N(0, sigma), encoded in fmt, expert-major."""
    nbytes = n_expert * tensor_bytes(fmt, n_rows * n_in)
    out = np.empty(nbytes, dtype=np.uint8)
    cb = None
    if fmt == CB2:
        cb = np.ascontiguousarray(codebook, dtype=np.int8)
    got = _load().sy_gen_expert_tensor(fmt, seed, layer, tag, n_expert, n_rows, n_in, sigma,
                                       _ptr(cb) if cb is not None else None, _ptr(out),
                                       nthreads or default_threads())
    if got != nbytes:
        raise RuntimeError("synth: tensor generation failed (%d != %d)" % (got, nbytes))
    return out


def normal(seed, layer, tag, idx, n, sigma=1.0, first=0):
    out = np.empty(n, dtype=np.float32)
    _load().sy_gen_normal(seed, layer, tag, idx, first, n, sigma, _ptr(out))
    return out


def uniform(seed, layer, tag, idx, n, first=0):
    out = np.empty(n, dtype=np.float64)
    _load().sy_gen_uniform(seed, layer, tag, idx, first, n, _ptr(out))
    return out


def codebook(seed):
    out = np.empty((256, 8), dtype=np.int8)
    _load().sy_gen_codebook(seed, TAG_CODEBOOK, _ptr(out))
    return out


def to_bf16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().sy_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def to_f16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().sy_f32_to_f16(_ptr(x), x.size, _ptr(out))
    return out


@dataclass
class Layer:
    """One MoE layer's weights as host arrays (bytes for block formats)."""
    n_embd: int
    n_expert: int
    n_expert_used: int
    n_ff_exp: int
    n_ff_shared: int
    gate_fmt: int
    up_fmt: int
    down_fmt: int
    shared_fmt: int
    router_w: np.ndarray                     # [E][D] fp32, row e = expert e
    gate: np.ndarray                         # [E][F][D] blocks
    up: np.ndarray
    down: np.ndarray                         # [E][D][F] blocks
    sh_gate: Optional[np.ndarray] = None     # [Fs][D]
    sh_up: Optional[np.ndarray] = None
    sh_down: Optional[np.ndarray] = None     # [D][Fs]
    router_bias: Optional[np.ndarray] = None  # [E] fp32
    route_scale: float = 1.0
    codebook: Optional[np.ndarray] = None    # [256][8] int8
    gamma: Optional[np.ndarray] = None       # [D] fp32 (RMSNorm weight, stack only)

    def expert_bytes(self):
        D, F = self.n_embd, self.n_ff_exp
        return (tensor_bytes(self.gate_fmt, F * D) + tensor_bytes(self.up_fmt, F * D)
                + tensor_bytes(self.down_fmt, D * F))

    def shared_bytes(self):
        if not self.n_ff_shared:
            return 0
        return 3 * tensor_bytes(self.shared_fmt, self.n_ff_shared * self.n_embd)


def make_layer(seed, layer, D, E, k, F, Fs, gate_fmt=Q2K, down_fmt=Q2K, shared_fmt=Q8_0, cb=None,
               gamma=False, nthreads=None, route_scale=1.0):
    """A layer of N(0, 0.02) weights encoded in the given formats."""
    nt = nthreads or default_threads()
    kw = dict(codebook=cb, nthreads=nt)
    L = Layer(
        n_embd=D, n_expert=E, n_expert_used=k, n_ff_exp=F, n_ff_shared=Fs,
        gate_fmt=gate_fmt, up_fmt=gate_fmt, down_fmt=down_fmt, shared_fmt=shared_fmt,
        router_w=normal(seed, layer, TAG_ROUTER, 0, D * E, WEIGHT_SIGMA).reshape(E, D),
        gate=expert_tensor(gate_fmt, seed, layer, TAG_GATE, E, F, D, **kw),
        up=expert_tensor(gate_fmt, seed, layer, TAG_UP, E, F, D, **kw),
        down=expert_tensor(down_fmt, seed, layer, TAG_DOWN, E, D, F, **kw),
        route_scale=route_scale, codebook=cb,
    )
    if Fs:
        L.sh_gate = expert_tensor(shared_fmt, seed, layer, TAG_SH_GATE, 1, Fs, D, **kw)
        L.sh_up = expert_tensor(shared_fmt, seed, layer, TAG_SH_UP, 1, Fs, D, **kw)
        L.sh_down = expert_tensor(shared_fmt, seed, layer, TAG_SH_DOWN, 1, D, Fs, **kw)
    if gamma:
        u = uniform(seed, layer, TAG_GAMMA, 0, D)
        L.gamma = (0.9 + 0.2 * u).astype(np.float32)
    return L


def activations(seed, T, D, layer=0):
    """x ~ N(0, 1), [T][D] fp32."""
    return normal(seed, layer, TAG_X, 0, T * D, 1.0).reshape(T, D)


def zipf_bias(seed, E, s=1.1):
    """bias_e = ln p_rank(e) with p_r proportional to r^-s, ranks from a seeded
    Fisher-Yates shuffle of the experts (a hot-expert skew)."""
    u = uniform(seed, 0, TAG_PERM, 0, E)
    perm = np.arange(E)
    for i in range(E - 1, 0, -1):
        j = int(u[i] * (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    bias = np.empty(E, dtype=np.float32)
    bias[perm] = np.log(p).astype(np.float32)  # expert perm[i] has rank i+1
    return bias


# ---- the five workloads -----------------------------------------------------

DS4_FLASH = dict(D=4096, E=256, k=6, F=2048, Fs=2048, n_layer=43)
WEIGHTS_SEED = 1  # decode_b1, decode_b32 and prefill_2048 run on the same layer


@dataclass
class Workload:
    name: str
    T: int
    mode: int                 # F32 or BF16 activations
    layers: list = field(default_factory=list)
    x: Optional[np.ndarray] = None        # [T][D] fp32 (F32 mode)
    x_bf16: Optional[np.ndarray] = None   # [T][D] bf16 bits (BF16 mode)
    n_layer: int = 1
    eps: float = 1e-6


def tiny():
    L = make_layer(0, 0, D=256, E=16, k=2, F=128, Fs=0)
    return Workload("tiny", 4, F32, [L], x=activations(0, 4, 256))


def flash_layer(nthreads=None):
    s = DS4_FLASH
    return make_layer(WEIGHTS_SEED, 0, D=s["D"], E=s["E"], k=s["k"], F=s["F"], Fs=s["Fs"],
                      nthreads=nthreads)


def decode_b1(layer=None, nthreads=None):
    L = layer or flash_layer(nthreads)
    return Workload("decode_b1", 1, F32, [L], x=activations(1, 1, L.n_embd))


def decode_b32(layer=None, nthreads=None):
    L = layer or flash_layer(nthreads)
    import copy
    Lb = copy.copy(L)
    Lb.router_bias = zipf_bias(2, L.n_expert)
    return Workload("decode_b32_zipf", 32, F32, [Lb], x=activations(2, 32, L.n_embd))


def prefill_2048(layer=None, nthreads=None, T=2048):
    L = layer or flash_layer(nthreads)
    x = activations(3, T, L.n_embd)
    return Workload("prefill_2048", T, BF16, [L], x_bf16=to_bf16_bits(x))


def stack_layer(l, cb, nthreads=None, E=None):
    s = DS4_FLASH
    return make_layer(4, l, D=s["D"], E=E or s["E"], k=s["k"], F=s["F"], Fs=s["Fs"], gate_fmt=CB2,
                      down_fmt=Q2K, shared_fmt=Q8_0, cb=cb, gamma=True, nthreads=nthreads)


def stack_layer_sampled(l, cb, nthreads=None):
    """One block of the stack with every expert and shared tensor drawn as
    random codes (sampled_tensor: each field uniform, block scales set for a
    weight spread near the N(0, 0.02) of the quantized recipe): the formats,
    shapes and byte counts of stack_layer without running the encoders (the
    codebook encoder takes minutes per full layer).  Router and RMSNorm
    weights as in stack_layer."""
    s = DS4_FLASH
    D, E, k, F, Fs = s["D"], s["E"], s["k"], s["F"], s["Fs"]
    nt = nthreads or default_threads()
    L = Layer(
        n_embd=D, n_expert=E, n_expert_used=k, n_ff_exp=F, n_ff_shared=Fs,
        gate_fmt=CB2, up_fmt=CB2, down_fmt=Q2K, shared_fmt=Q8_0,
        router_w=normal(4, l, TAG_ROUTER, 0, D * E, WEIGHT_SIGMA).reshape(E, D),
        gate=sampled_tensor(CB2, 4, l, TAG_GATE, E, F, D, codebook=cb, nthreads=nt),
        up=sampled_tensor(CB2, 4, l, TAG_UP, E, F, D, codebook=cb, nthreads=nt),
        down=sampled_tensor(Q2K, 4, l, TAG_DOWN, E, D, F, nthreads=nt),
        codebook=cb,
    )
    L.sh_gate = sampled_tensor(Q8_0, 4, l, TAG_SH_GATE, 1, Fs, D, nthreads=nt)
    L.sh_up = sampled_tensor(Q8_0, 4, l, TAG_SH_UP, 1, Fs, D, nthreads=nt)
    L.sh_down = sampled_tensor(Q8_0, 4, l, TAG_SH_DOWN, 1, D, Fs, nthreads=nt)
    L.gamma = (0.9 + 0.2 * uniform(4, l, TAG_GAMMA, 0, D)).astype(np.float32)
    return L


def stack43(B=1, n_layer=43, nthreads=None, layer_fn=None):
    """The 43-block stack; layers are generated one by one through layer_fn
    (default: keep them all in host memory)."""
    cb = codebook(4)
    x = activations(4, B, DS4_FLASH["D"], layer=B)
    wl = Workload("stack43_b%d" % B, B, F32, [], x=x, n_layer=n_layer)
    wl.codebook = cb
    return wl


def sampled_tensor(fmt, seed, layer, tag, n_expert, n_rows, n_in, sigma=WEIGHT_SIGMA, codebook=None,
                   nthreads=None):
    """n_expert matrices whose blocks are drawn directly as random codes (every
    field uniform, block scale set for a weight std near sigma), expert-major."""
    nbytes = n_expert * tensor_bytes(fmt, n_rows * n_in)
    out = np.empty(nbytes, dtype=np.uint8)
    cb = None
    if fmt == CB2:
        cb = np.ascontiguousarray(codebook, dtype=np.int8)
    lib = _load()
    fn = lib.sy_sample_expert_tensor
    fn.restype = ctypes.c_int64
    fn.argtypes = lib.sy_gen_expert_tensor.argtypes
    got = fn(fmt, seed, layer, tag, n_expert, n_rows, n_in, sigma, _ptr(cb) if cb is not None else None,
             _ptr(out), nthreads or default_threads())
    if got != nbytes:
        raise RuntimeError("synth: sampled tensor failed (%d != %d)" % (got, nbytes))
    return out
