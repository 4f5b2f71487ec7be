"""Seeded synthetic inputs for the sparse MoE layer.

This module is shared by the CPU oracle tests and the GPU path. It only draws
random numbers and stores them in the weight formats the layer accepts (fp32,
or bf16 bit patterns rounded to nearest-even). It holds none of the layer's
arithmetic: no routing, no quantization, no matrix products.

Shapes follow the Qwen3-Next layer statement on the Red Lite "Architecture"
page (section "Qwen3-Next shape": hidden 2048, 512 routed experts, top-10, one
shared expert, expert intermediate 512). The pages measure on real GGUF files
and chat prompts; seeded normal draws of the same shapes stand in for them.

Seeding: one NumPy PCG64 stream per tensor, keyed by
``[20261203 + 100*config, stream, expert, matrix]``. Streams: 0 router,
1 shared-gate vector, 2 routed experts, 3 shared expert, 4 activations x,
5 router bias, 6 the pre-MoE norm's gamma (multi-layer stacks). Every expert matrix has its own stream, so any single expert
can be regenerated without drawing the others.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

SEED_BASE = 20261203

STREAM_ROUTER = 0
STREAM_GATEVEC = 1
STREAM_EXPERTS = 2
STREAM_SHARED = 3
STREAM_X = 4
STREAM_BIAS = 5
STREAM_NORM = 6

MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2


# Expert formats stored as 32-weight blocks of 2-, 3- or 4-bit codes.
BLOCK_FORMATS = ("q2", "q3", "q4")


@dataclass(frozen=True)
class LayerConfig:
    """Shape, weight formats and draw parameters of one MoE layer workload."""
    name: str
    index: int            # seed namespace (0..4 for the five standard workloads)
    H: int                # hidden
    E: int                # routed experts
    K: int                # experts per token
    I: int                # routed expert intermediate
    Is: int               # shared expert intermediate
    T: int                # rows of x in the workload
    rows_per_call: int    # rows handed to one forward call (1 = decode)
    router_t: str         # "f32" | "bf16"
    expert_t: str         # "f32" | "bf16" | "q2" | "q3" | "q4"
    shared_t: str         # "f32" | "bf16"
    router_std: float
    expert_std: float = 0.02
    bias_std: float = 0.0  # 0 = no router bias
    x_std: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return SEED_BASE + 100 * self.index

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# The five workloads. The tiny one is small enough for the oracle to finish in
# well under a second; the others use the full Qwen3-Next layer shape.
CONFIGS = {
    0: LayerConfig("tiny_fp32", 0, H=512, E=64, K=4, I=128, Is=128, T=1, rows_per_call=1,
                   router_t="f32", expert_t="f32", shared_t="f32", router_std=0.05),
    1: LayerConfig("decode_bf16", 1, H=2048, E=512, K=10, I=512, Is=512, T=1000, rows_per_call=1,
                   router_t="bf16", expert_t="bf16", shared_t="bf16", router_std=0.03),
    2: LayerConfig("decode_q2", 2, H=2048, E=512, K=10, I=512, Is=512, T=1000, rows_per_call=1,
                   router_t="bf16", expert_t="q2", shared_t="bf16", router_std=0.03),
    3: LayerConfig("fewrow_q2", 3, H=2048, E=512, K=10, I=512, Is=512, T=1000, rows_per_call=2,
                   router_t="bf16", expert_t="q2", shared_t="bf16", router_std=0.03),
    4: LayerConfig("prefill_q2", 4, H=2048, E=512, K=10, I=512, Is=512, T=2048, rows_per_call=2048,
                   router_t="bf16", expert_t="q2", shared_t="bf16", router_std=0.03, bias_std=1.0),
}


def _rng(cfg: LayerConfig, stream: int, *key: int) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, stream, *key])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the 16-bit patterns.

    Storage-format conversion of inputs (bf16 weights are stored this way);
    inputs are finite normal draws, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if fmt == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(fmt)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def expert_matrix_f32(cfg: LayerConfig, e: int, mat: int) -> np.ndarray:
    """Routed expert ``e`` matrix as fp32 values.

    gate/up are [I][H], down is [H][I]. For bf16 and block-format (q2, q3,
    q4) experts the draw is rounded to bf16 first, so the block workloads
    quantize exactly the values the bf16 workload stores (same seed namespace
    rule as the bf16 case).
    """
    shape = (cfg.I, cfg.H) if mat in (MAT_GATE, MAT_UP) else (cfg.H, cfg.I)
    a = _normal(_rng(cfg, STREAM_EXPERTS, e, mat), shape, cfg.expert_std)
    if cfg.expert_t == "bf16" or cfg.expert_t in BLOCK_FORMATS:
        a = bf16_bits_to_f32(f32_to_bf16_bits(a)).reshape(shape)
    return a


def expert_matrix_stored(cfg: LayerConfig, e: int, mat: int) -> np.ndarray:
    """Routed expert matrix in its storage format (f32 values or bf16 bits).

    Block-format experts are returned as their fp32 source; packing belongs to
    the consumer (the library packer or the oracle's own quantizer).
    """
    shape = (cfg.I, cfg.H) if mat in (MAT_GATE, MAT_UP) else (cfg.H, cfg.I)
    a = _normal(_rng(cfg, STREAM_EXPERTS, e, mat), shape, cfg.expert_std)
    if cfg.expert_t == "bf16":
        return f32_to_bf16_bits(a)
    if cfg.expert_t in BLOCK_FORMATS:
        return bf16_bits_to_f32(f32_to_bf16_bits(a)).reshape(shape)
    return a


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def expert_stacks(cfg: LayerConfig, experts=None):
    """Stacked routed-expert weights (gate [E][I][H], up [E][I][H], down [E][H][I]).

    f32/bf16 workloads only (block-format stacks are packed matrix by matrix
    by the consumer). ``experts`` restricts generation to a subset (others are zero).
    """
    assert cfg.expert_t in ("f32", "bf16")
    dt = np.float32 if cfg.expert_t == "f32" else np.uint16
    g = np.zeros((cfg.E, cfg.I, cfg.H), dt)
    u = np.zeros((cfg.E, cfg.I, cfg.H), dt)
    d = np.zeros((cfg.E, cfg.H, cfg.I), dt)
    todo = range(cfg.E) if experts is None else sorted(set(int(e) for e in experts))

    def fill(e):
        g[e] = expert_matrix_stored(cfg, e, MAT_GATE)
        u[e] = expert_matrix_stored(cfg, e, MAT_UP)
        d[e] = expert_matrix_stored(cfg, e, MAT_DOWN)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, todo))
    return g, u, d


def dense_weights(cfg: LayerConfig) -> dict:
    """Router, shared-gate vector, optional bias and the shared expert."""
    out = {}
    out["router_w"] = _store(_normal(_rng(cfg, STREAM_ROUTER), (cfg.E, cfg.H), cfg.router_std), cfg.router_t)
    # The shared-gate vector uses the router's spread and storage format.
    out["gate_vec"] = _store(_normal(_rng(cfg, STREAM_GATEVEC), (cfg.H,), cfg.router_std), cfg.router_t)
    out["router_bias"] = (_normal(_rng(cfg, STREAM_BIAS), (cfg.E,), cfg.bias_std)
                          if cfg.bias_std > 0 else None)
    out["sh_gate"] = _store(_normal(_rng(cfg, STREAM_SHARED, 0), (cfg.Is, cfg.H), cfg.expert_std), cfg.shared_t)
    out["sh_up"] = _store(_normal(_rng(cfg, STREAM_SHARED, 1), (cfg.Is, cfg.H), cfg.expert_std), cfg.shared_t)
    out["sh_down"] = _store(_normal(_rng(cfg, STREAM_SHARED, 2), (cfg.H, cfg.Is), cfg.expert_std), cfg.shared_t)
    return out


def norm_weights(cfg: LayerConfig, layer: int = 0) -> np.ndarray:
    """gamma[H] of a layer's pre-MoE RMS norm: 1 + N(0, 0.1) in fp32 (a
    trained norm scale near one)."""
    g = _normal(_rng(cfg, STREAM_NORM, layer), (cfg.H,), 0.1)
    g += np.float32(1.0)
    return g


def activations(cfg: LayerConfig, T: int | None = None, instance: int = 0) -> np.ndarray:
    """x[T][H] ~ N(0, x_std) in fp32; ``instance`` selects an independent draw."""
    T = cfg.T if T is None else T
    return _normal(_rng(cfg, STREAM_X, instance), (T, cfg.H), cfg.x_std)


def layer_instance(cfg: LayerConfig, instance: int) -> LayerConfig:
    """A distinct layer of the same shape (router, gate vector and shared expert
    redrawn), used to rotate through several layers' dense weights."""
    if instance == 0:
        return cfg
    return cfg.with_(name=f"{cfg.name}#{instance}", index=cfg.index + 1000 * instance)
