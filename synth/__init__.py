"""Seeded synthetic inputs for the block-scaled FP4 MoE layer.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It draws random source tensors, converts them to bfloat16 bit
patterns and computes the router's top-k selection (routing is done by the
caller of the MoE layer, so both sides must consume the same ids and
weights).  It holds none of the quantization or FFN arithmetic.

Workload shapes follow the model cards on block_scaled_fp4_nvfp4: 512 routed
experts, hidden 2560, expert intermediate 640 (gate_up 1280 x 2560, down
2560 x 640), 48 layers, top-10 routing (top-5 in the "FP4-Local AZ" card's
table of differences), a 1280-wide shared expert with a bf16 gate (same
card, "The shared expert"), 16 concurrent sequences and 8K prefill
("Measured on 2 x DGX Spark", QAD5500-Hybrid card).  No dataset or real
checkpoint is used; every value is drawn here from a fixed seed.

Seeding: numpy PCG64 seeded by SeedSequence(entropy=<seed>, spawn_key=<key>),
with key = (stream, ...).  Streams: 0 routed weights (layer, expert, proj
with 0 gate / 1 up / 2 down), 1 activations, 2 router logits, 3 router bias,
4 shared-expert weights (proj 0 gate / 1 up / 2 down), 5 shared-expert gate
vector, 6 outlier rows of the streaming workload, 7 calibration activations,
8 calibration row counts.  Values are drawn in
float32 and rounded to bfloat16 by round-to-nearest-even.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

__all__ = [
    "MoEConfig", "CONFIGS", "FP8_ROUTED_LAYERS", "stack_configs", "rng", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "normal_bf16", "expert_weights", "layer_weights", "activations",
    "router_logits", "router_bias", "route", "routing", "shared_expert",
    "streaming_expert", "calibration_hessian", "calibration_rows",
]

STREAM_WEIGHTS, STREAM_X, STREAM_LOGITS, STREAM_BIAS, STREAM_SHARED, \
    STREAM_SHARED_GATE, STREAM_OUTLIERS, STREAM_CALIB, STREAM_CALIB_ROWS = range(9)
WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One routed-expert layer workload (sizes, formats, seeds)."""
    name: str
    num_experts: int
    top_k: int
    hidden: int
    inter: int
    tokens: int
    w_fmt: str            # "nvfp4" | "mxfp4" | "fp8_block"
    a_fmt: str            # "none" | "nvfp4" | "mxfp8" | "fp8_row"
    rule: str = "4over6"  # weight block-scale rule: "4over6" | "rtn"
    router_bias: bool = False
    shared_inter: int = 0  # 0: no shared expert
    weight_seed: int = 2   # configs of the same expert shapes share weights
    input_seed: int = 2

    @property
    def pairs(self) -> int:
        return self.tokens * self.top_k

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # tiny layer: 8 experts, top-2, hidden 256, intermediate 128, 64 tokens
    "tiny": MoEConfig("tiny", 8, 2, 256, 128, 64, "nvfp4", "none",
                      weight_seed=1, input_seed=1),
    # decode: 512 experts, top-10, 16 tokens, NVFP4 weights, bf16 activations
    "decode": MoEConfig("decode", 512, 10, 2560, 640, 16, "nvfp4", "none",
                        input_seed=2),
    # prefill: top-5, 8192 tokens, NVFP4 x NVFP4, biased router, MXFP8 shared expert
    "prefill_nvfp4": MoEConfig("prefill_nvfp4", 512, 5, 2560, 640, 8192,
                               "nvfp4", "nvfp4", router_bias=True,
                               shared_inter=1280, input_seed=3),
    # prefill: top-10, 8192 tokens, MXFP4 weights x dynamic MXFP8 activations
    "prefill_mxfp4": MoEConfig("prefill_mxfp4", 512, 10, 2560, 640, 8192,
                               "mxfp4", "mxfp8", input_seed=4),
    # same inputs through the block-FP8 copy of the layer
    "prefill_fp8": MoEConfig("prefill_fp8", 512, 10, 2560, 640, 8192,
                             "fp8_block", "fp8_row", input_seed=4),
}


# The mixed-precision 48-layer routed-expert stack of the MXFP4-FP8-R12 card
# ("Quantization format", "Retained layers"): these zero-based layers keep
# block-FP8 experts with dynamic FP8 activations, the other 36 run MXFP4 x
# dynamic MXFP8.
FP8_ROUTED_LAYERS = (19, 20, 21, 23, 28, 32, 33, 40, 41, 43, 44, 45)


def stack_configs(n_layers: int = 48, tokens: int = 16, num_experts: int = 512, top_k: int = 10,
                  hidden: int = 2560, inter: int = 640, fp8_layers=FP8_ROUTED_LAYERS):
    """Per-layer configurations of the decode stack (seeds differ per layer)."""
    out = []
    for l in range(n_layers):
        fp8 = l in fp8_layers
        out.append(MoEConfig(f"stack{l}", num_experts, top_k, hidden, inter, tokens,
                             "fp8_block" if fp8 else "mxfp4", "fp8_row" if fp8 else "mxfp8",
                             weight_seed=100 + l, input_seed=300 + l))
    return out


def rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key))))


def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(gen: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    v = gen.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


def expert_weights(cfg: MoEConfig, e: int, layer: int = 0):
    """bf16 bits of one expert: fused gate_up [2I, H] (gate rows first), down [H, I]."""
    I, H = cfg.inter, cfg.hidden
    gate = normal_bf16(rng(cfg.weight_seed, STREAM_WEIGHTS, layer, e, 0), (I, H), WEIGHT_STD)
    up = normal_bf16(rng(cfg.weight_seed, STREAM_WEIGHTS, layer, e, 1), (I, H), WEIGHT_STD)
    down = normal_bf16(rng(cfg.weight_seed, STREAM_WEIGHTS, layer, e, 2), (H, I), WEIGHT_STD)
    return np.concatenate([gate, up], axis=0), down


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def layer_weights(cfg: MoEConfig, layer: int = 0, experts=None):
    """bf16 bits of a whole layer: W13 [E, 2I, H], W2 [E, H, I] (threaded draw)."""
    ids = list(range(cfg.num_experts)) if experts is None else list(experts)
    I, H = cfg.inter, cfg.hidden
    w13 = np.empty((len(ids), 2 * I, H), np.uint16)
    w2 = np.empty((len(ids), H, I), np.uint16)

    def fill(j):
        a, b = expert_weights(cfg, ids[j], layer)
        w13[j] = a
        w2[j] = b

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(ids))))
    return w13, w2


def activations(cfg: MoEConfig) -> np.ndarray:
    """bf16 bits of x [T, H], N(0, 1)."""
    return normal_bf16(rng(cfg.input_seed, STREAM_X), (cfg.tokens, cfg.hidden))


def router_logits(cfg: MoEConfig) -> np.ndarray:
    return rng(cfg.input_seed, STREAM_LOGITS).standard_normal(
        (cfg.tokens, cfg.num_experts), dtype=np.float32)


def router_bias(cfg: MoEConfig) -> np.ndarray:
    if not cfg.router_bias:
        return np.zeros(cfg.num_experts, np.float32)
    return rng(cfg.input_seed, STREAM_BIAS).standard_normal(cfg.num_experts, dtype=np.float32)


def route(logits: np.ndarray, bias: np.ndarray, k: int):
    """Top-k routing done by the caller of the layer.

    l' = fp32(logit + bias); the k largest l' are selected (equal values: lower
    expert id first); weights are the softmax over the k selected l' (i.e. the
    renormalized top-k softmax), computed in float64 and rounded to float32.
    """
    lp = (logits.astype(np.float32) + bias.astype(np.float32)[None, :]).astype(np.float32)
    order = np.argsort(-lp, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(lp, order, axis=1).astype(np.float64)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def routing(cfg: MoEConfig):
    return route(router_logits(cfg), router_bias(cfg), cfg.top_k)


def shared_expert(cfg: MoEConfig):
    """bf16 bits of the shared expert: fused gate_up [2S, H], down [H, S], gate vector [H]."""
    S, H = cfg.shared_inter, cfg.hidden
    g = normal_bf16(rng(cfg.weight_seed, STREAM_SHARED, 0), (S, H), WEIGHT_STD)
    u = normal_bf16(rng(cfg.weight_seed, STREAM_SHARED, 1), (S, H), WEIGHT_STD)
    d = normal_bf16(rng(cfg.weight_seed, STREAM_SHARED, 2), (H, S), WEIGHT_STD)
    wg = normal_bf16(rng(cfg.weight_seed, STREAM_SHARED_GATE), (H,), WEIGHT_STD)
    return np.concatenate([g, u], axis=0), d, wg


def streaming_expert(layer: int, e: int, hidden: int = 2560, inter: int = 640,
                     seed: int = 5):
    """Heavy-tailed source weights of the streaming-quantization workload.

    Student-t (nu = 4) scaled to standard deviation 0.02 (t_4 has variance 2),
    with round(1% of rows) rows of each of gate, up and down (chosen without
    replacement) multiplied by 8, rounded to bf16.  Returns (W13 [2I,H], W2 [H,I]).
    """
    outs = []
    for proj, shape in ((0, (inter, hidden)), (1, (inter, hidden)), (2, (hidden, inter))):
        g = rng(seed, STREAM_WEIGHTS, layer, e, proj)
        v = (g.standard_t(4, shape) * (WEIGHT_STD / np.sqrt(2.0))).astype(np.float32)
        rows = rng(seed, STREAM_OUTLIERS, layer, e, proj).choice(
            shape[0], size=int(round(0.01 * shape[0])), replace=False)
        v[rows] *= np.float32(8.0)
        outs.append(f32_to_bf16_bits(v))
    return np.concatenate(outs[:2], axis=0), outs[2]


def calibration_rows(seed: int, num_experts: int) -> np.ndarray:
    """Calibration rows routed to each expert (int32 [E]): log-normal around
    the median of 5,007 rows per expert that the Local-Hessian card reports
    ("Calibration data"), at least 64, except one expert with no rows and one
    with 30 (the card's thin experts, which keep plain-max scales)."""
    g = rng(seed, STREAM_CALIB_ROWS)
    n = np.maximum(64, np.round(5007.0 * np.exp(0.8 * g.standard_normal(num_experts)))).astype(np.int32)
    if num_experts >= 4:
        n[1] = 0
        n[2] = 30
    return n


def calibration_hessian(seed: int, expert: int, in_dim: int, n_rows: int, proj: int = 0) -> np.ndarray:
    """Synthetic local Hessian blocks of one expert matrix's input: n_rows
    calibration activation rows a_t (bf16 values; per-channel scales
    log-normal with sigma 0.5; within each 16-column block a shared
    component of weight c_b ~ U(0, 1), so the blocks are correlated), and
    H_b = (1/n) sum_t a_t,b a_t,b^T over the 16 columns of block b, summed in
    float64 and rounded to float32.  Returns float32 [in_dim/16, 16, 16];
    zeros when n_rows == 0."""
    nb = in_dim // 16
    if n_rows == 0:
        return np.zeros((nb, 16, 16), np.float32)
    g = rng(seed, STREAM_CALIB, expert, proj)
    scale = np.exp(0.5 * g.standard_normal(in_dim)).astype(np.float32)
    c = g.uniform(0.0, 1.0, nb).astype(np.float32)
    z = g.standard_normal((n_rows, in_dim), dtype=np.float32)
    sh = g.standard_normal((n_rows, nb), dtype=np.float32)
    a = (z + np.repeat(c[None, :] * sh, 16, axis=1)) * scale[None, :]
    a = bf16_bits_to_f32(f32_to_bf16_bits(a)).astype(np.float64).reshape(n_rows, nb, 16)
    return (np.einsum("tbi,tbj->bij", a, a) / n_rows).astype(np.float32)
