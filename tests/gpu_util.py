"""Helpers shared by the GPU tests: device upload of bf16 bit patterns,
quantization of a layer through the C ABI, oracle-side layers.

GPU layers are quantized by the library (fp4_quantize); oracle layers are
quantized by the oracle from the same bf16 source.  The two never exchange
values: tests compare them."""
import functools
import os

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")


def gpu_ok() -> bool:
    return torch.cuda.is_available()


def dev_bf16(bits: np.ndarray) -> "torch.Tensor":
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: "torch.Tensor") -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def print_case(msg: str):
    print(f"[case] {msg}", flush=True)


def gpu_layer(cfg, w13_bits, w2_bits, shared=None, rule=None):
    """Quantize bf16 weights on the GPU through fp4_quantize; returns MoELayer."""
    from block_scaled_fp4_nvfp4_amd import MoELayer, quantize
    rule = rule or cfg.rule
    w13 = dev_bf16(w13_bits)
    q13 = quantize(w13, cfg.w_fmt, rule)
    del w13
    w2 = dev_bf16(w2_bits)
    q2 = quantize(w2, cfg.w_fmt, rule)
    del w2
    E, I2, H = w13_bits.shape
    layer = MoELayer(cfg.w_fmt, cfg.a_fmt, E, H, I2 // 2, cfg.top_k,
                     q13["codes"], q13["scales"], q2["codes"], q2["scales"],
                     q13["tensor_scale"], q2["tensor_scale"])
    if shared is not None:
        s13, s2, gate = shared
        a = quantize(dev_bf16(s13), "mxfp8")
        b = quantize(dev_bf16(s2), "mxfp8")
        layer.shared_inter = s13.shape[0] // 2
        layer.ws13, layer.ws13_scale = a["codes"], a["scales"]
        layer.ws2, layer.ws2_scale = b["codes"], b["scales"]
        layer.shared_gate = dev_bf16(gate)
    return layer


class OracleLayer:
    """Oracle-side layer quantizing experts lazily (only those a test touches)."""

    def __init__(self, cfg, w13_bits, w2_bits, shared=None, rule=None):
        from oracle import moe
        self.cfg, self.rule = cfg, rule or cfg.rule
        self.w13_bits, self.w2_bits = w13_bits, w2_bits
        self._moe = moe
        self.shared = None
        if shared is not None:
            s13, s2, gate = shared
            self.shared = dict(w13=moe.quantize_expert_weight(s13, "mxfp8"),
                               w2=moe.quantize_expert_weight(s2, "mxfp8"), gate_bits=gate)

    _done = None

    def prefetch(self, experts, processes=16):
        """Quantize these experts now, in a pool of processes (the oracle is
        plain single-threaded numpy; a whole decode layer's touched experts
        take minutes on one core)."""
        import concurrent.futures as cf
        import multiprocessing as mp

        from oracle_pool import quantize_expert_pair
        if self._done is None:
            self._done = {}
        todo = [int(e) for e in experts if int(e) not in self._done]
        tasks = [(self.w13_bits[e], self.w2_bits[e], self.cfg.w_fmt, self.rule) for e in todo]
        with cf.ProcessPoolExecutor(max(1, min(processes, len(todo))), mp.get_context("spawn")) as ex:
            for e, r in zip(todo, ex.map(quantize_expert_pair, tasks)):
                self._done[e] = r

    def w13(self, e):
        if self._done is not None and e in self._done:
            return self._done[e][0]
        return self._w13(e)

    def w2(self, e):
        if self._done is not None and e in self._done:
            return self._done[e][1]
        return self._w2(e)

    @functools.lru_cache(maxsize=None)
    def _w13(self, e):
        return self._moe.quantize_expert_weight(self.w13_bits[e], self.cfg.w_fmt, self.rule)

    @functools.lru_cache(maxsize=None)
    def _w2(self, e):
        return self._moe.quantize_expert_weight(self.w2_bits[e], self.cfg.w_fmt, self.rule)

    def as_dict(self):
        d = dict(w_fmt=self.cfg.w_fmt, a_fmt=self.cfg.a_fmt, num_experts=self.w13_bits.shape[0],
                 hidden=self.w13_bits.shape[2], inter=self.w13_bits.shape[1] // 2,
                 w13=self.w13, w2=self.w2)
        if self.shared is not None:
            d["shared"] = self.shared
        return d


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
