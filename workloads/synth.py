"""Seeded synthetic inputs for the MoE expert path.

This module only draws random inputs and stores them in the formats the two
sides consume (fp32, or bf16 as raw 16-bit patterns).  It holds none of the
layer's arithmetic: no routing, no gating, no capacity rule, no FFN.  Both the
CPU oracle and the GPU path take their inputs from here, bit for bit.

Shapes follow the five workloads the method is studied on:
  * a tiny fp32 layer (T64 d128 f256 E8 k2, softmax gates),
  * a Mixtral-shaped bf16 prefill layer (T4096 d4096 f14336 E8 k2) whose
    router logits are produced from x and an fp32 gate matrix,
  * a DeepSeek-V3-shaped bf16 decode layer (T128 d7168 f2048 E256 k8,
    sigmoid gates),
  * the same DeepSeek-V3 shape at prefill scale (T8192) with a Zipf-like
    popularity bias added to the logits,
  * one expert-parallel rank's share (T16384 d4096 f1536, E128 global of
    which experts [0,32) are local, k2, capacity factor 1.25) with a
    per-expert N(0, 0.5) logit bias.

Random streams: numpy PCG64 generators seeded by independent children of
SeedSequence(seed): one child each for x, logits, bias and the gate matrix,
and one child per expert (so any expert's weights can be regenerated alone).
N(mu, s) means standard deviation s.  Normals are drawn in fp32, scaled by s
in fp32, and bf16 values are obtained by round-to-nearest-even on the fp32
bit pattern.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, Optional, Tuple

import numpy as np

GATE_SOFTMAX = "softmax_topk_renorm"
GATE_SIGMOID = "sigmoid_topk_norm"

# child indices of the workload's SeedSequence
_X, _LOGITS, _BIAS, _WGATE, _EXPERTS = range(5)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(ss: np.random.SeedSequence, shape, std: float, out_dtype: str) -> np.ndarray:
    """Draw N(0, std) in fp32 from one stream; out_dtype 'f32' or 'bf16'."""
    g = np.random.Generator(np.random.PCG64(ss))
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if out_dtype == "bf16":
        return f32_to_bf16_bits(a).reshape(shape)
    return a


@dataclasses.dataclass
class Workload:
    """One seeded MoE-layer input set.

    x:        [T, d]  float32 (dtype 'f32') or uint16 bf16 bits (dtype 'bf16')
    logits:   [T, E]  float32, or None when the logits come from x and w_gate
    w_gate:   [d, E]  float32 gate matrix (router-logits workloads only)
    Expert weights in the logical x.W layout, per expert e:
        W1[e], W3[e]: [d, f]; W2[e]: [f, d]   (same dtype as x)
    Only experts [e_begin, e_end) carry weights.
    """

    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    gate: str
    dtype: str
    capacity_factor: Optional[float]
    e_begin: int
    e_end: int
    seed: int
    x: np.ndarray
    logits: Optional[np.ndarray]
    w_gate: Optional[np.ndarray]
    _expert_ss: list = dataclasses.field(repr=False, default_factory=list)

    @property
    def E_loc(self) -> int:
        return self.e_end - self.e_begin

    def expert_weights(self, e: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(W1 [d,f], W3 [d,f], W2 [f,d]) of global expert e, regenerated from its own stream."""
        if not (self.e_begin <= e < self.e_end):
            raise ValueError(f"expert {e} is not local to [{self.e_begin},{self.e_end})")
        c1, c3, c2 = (_child(self._expert_ss[e], i) for i in range(3))
        s_in = 1.0 / math.sqrt(self.d)
        s_out = 1.0 / math.sqrt(self.f)
        w1 = _normal(c1, (self.d, self.f), s_in, self.dtype)
        w3 = _normal(c3, (self.d, self.f), s_in, self.dtype)
        w2 = _normal(c2, (self.f, self.d), s_out, self.dtype)
        return w1, w3, w2

    def stacked_weights(self, experts=None):
        """Stack (W1, W3, W2) over local experts (or the given global ids), threaded."""
        ids = list(range(self.e_begin, self.e_end)) if experts is None else list(experts)
        with ThreadPoolExecutor(_threads()) as ex:
            parts = list(ex.map(self.expert_weights, ids))
        return (np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                np.stack([p[2] for p in parts]))

    def for_each_expert(self, fn: Callable[[int, tuple], None], threads: Optional[int] = None):
        """Generate local experts in parallel and hand each to fn(e, weights) in expert order."""
        ids = list(range(self.e_begin, self.e_end))
        n = threads or _threads()
        with ThreadPoolExecutor(n) as ex:
            # bounded look-ahead keeps host memory at ~2n experts
            futs = {}
            nxt = 0
            for e in ids:
                while nxt < len(ids) and nxt < ids.index(e) + 2 * n:
                    futs[ids[nxt]] = ex.submit(self.expert_weights, ids[nxt])
                    nxt += 1
                fn(e, futs.pop(e).result())


def _child(ss: np.random.SeedSequence, i: int) -> np.random.SeedSequence:
    """The i-th child of ss, derived statelessly (SeedSequence.spawn is stateful)."""
    return np.random.SeedSequence(entropy=ss.entropy, spawn_key=tuple(ss.spawn_key) + (i,),
                                  pool_size=ss.pool_size)


def _seeds(seed: int, E: int):
    root = np.random.SeedSequence(seed)
    kids = [_child(root, i) for i in range(5)]
    experts = [_child(kids[_EXPERTS], e) for e in range(E)]
    return kids, experts


def custom(name: str = "custom", *, T: int, d: int, f: int, E: int, k: int,
           gate: str = GATE_SOFTMAX, dtype: str = "bf16", seed: int = 0,
           capacity_factor: Optional[float] = None, e_begin: int = 0,
           e_end: Optional[int] = None, logit_bias: Optional[str] = None,
           logits_from_gate: bool = False, gate_std: float = 0.02,
           zipf_s: float = 1.1, zipf_beta: float = 0.4, bias_std: float = 0.5) -> Workload:
    """Build a seeded workload of any shape.

    logit_bias: None, 'zipf' (bias_e = -beta * s * ln(e + 1)) or 'normal'
    (bias_e ~ N(0, bias_std)); the bias is added to N(0,1) logits in fp64 and
    the sum rounded to fp32.
    logits_from_gate: draw a [d, E] fp32 gate matrix N(0, gate_std) instead of
    logits; the logits are then the router product of x and that matrix.
    """
    if e_end is None:
        e_end = E
    kids, experts = _seeds(seed, E)
    x = _normal(kids[_X], (T, d), 1.0, dtype)
    logits = None
    w_gate = None
    if logits_from_gate:
        w_gate = _normal(kids[_WGATE], (d, E), gate_std, "f32")
    else:
        logits = _normal(kids[_LOGITS], (T, E), 1.0, "f32")
        if logit_bias == "zipf":
            bias = -zipf_beta * zipf_s * np.log(np.arange(E, dtype=np.float64) + 1.0)
            logits = (logits.astype(np.float64) + bias[None, :]).astype(np.float32)
        elif logit_bias == "normal":
            g = np.random.Generator(np.random.PCG64(kids[_BIAS]))
            bias = g.standard_normal(E, dtype=np.float32).astype(np.float64) * bias_std
            logits = (logits.astype(np.float64) + bias[None, :]).astype(np.float32)
        elif logit_bias is not None:
            raise ValueError(logit_bias)
    return Workload(name=name, T=T, d=d, f=f, E=E, k=k, gate=gate, dtype=dtype,
                    capacity_factor=capacity_factor, e_begin=e_begin, e_end=e_end,
                    seed=seed, x=x, logits=logits, w_gate=w_gate, _expert_ss=experts)


# The five named workloads.  Each entry: keyword arguments of custom().
WORKLOADS = {
    "tiny_fp32": dict(T=64, d=128, f=256, E=8, k=2, gate=GATE_SOFTMAX, dtype="f32"),
    "mixtral_prefill": dict(T=4096, d=4096, f=14336, E=8, k=2, gate=GATE_SOFTMAX,
                            dtype="bf16", logits_from_gate=True, gate_std=0.02),
    "dsv3_decode": dict(T=128, d=7168, f=2048, E=256, k=8, gate=GATE_SIGMOID, dtype="bf16"),
    "dsv3_prefill_zipf": dict(T=8192, d=7168, f=2048, E=256, k=8, gate=GATE_SIGMOID,
                              dtype="bf16", logit_bias="zipf", zipf_s=1.1, zipf_beta=0.4),
    "ep_rank_share": dict(T=16384, d=4096, f=1536, E=128, k=2, gate=GATE_SOFTMAX,
                          dtype="bf16", capacity_factor=1.25, e_begin=0, e_end=32,
                          logit_bias="normal", bias_std=0.5),
}


def output_grad(wl: Workload) -> np.ndarray:
    """A seeded output gradient dy [T, d] for the backward pass: N(0, 1) in the
    layer dtype, from its own stream (independent of every other input)."""
    ss = _child(np.random.SeedSequence(wl.seed), 5)
    return _normal(ss, (wl.T, wl.d), 1.0, wl.dtype)


def make(name: str, seed: int = 0, **overrides) -> Workload:
    """One of the named workloads (optionally with fields overridden, e.g. T)."""
    kw = dict(WORKLOADS[name])
    kw.update(overrides)
    return custom(name, seed=seed, **kw)
