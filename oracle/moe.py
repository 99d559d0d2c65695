"""Routed-expert MoE FFN in float64 (oracle; test infrastructure only).

What the layer computes, per token t with selected experts e_tj and routing
weights w_tj (j < k):

    y_t = sum_j w_tj * W2~[e_tj] @ Qh( SiLU(Wg~[e_tj] @ x~_t) * (Wu~[e_tj] @ x~_t) )
          (+ sigmoid(x_t . w_g) * shared(x_t)   when a shared expert is present)

with W~ the dequantized weights (exact values), x~ = Qx(x) and Qh the
dynamic activation quantizers of the mode: identity for bf16 activations
(W4A16, the weight-only NVFP4 mode of the dabsLabs NVFP4 card), NVFP4 with
tensor scale amax/2688 and plain amax/6 block scales (W4A4; LocalHessian-
Experts card, opening section), MXFP8 per 32 (MXFP4-FP8-R12 card, section
"Quantization format"), or FP8 with one fp32 scale per (row, 128 columns)
(the dynamic-FP8 path of the retained routed experts, same card, runtime
contract table; a_fmt "fp8_row").
The fused gate_up weight holds gate rows first, then up rows (dabsLabs card:
experts stored stacked as [512, out, in] with fused gate_up).  The shared
expert ("FP4-Local AZ", section "The shared expert") is MXFP8 with MXFP8
activations and a bf16 sigmoid gate on unquantized x.

Readings: routing weights are applied after the down projection (in the
combine); the intermediate h stays float64 here (float32 on the GPU) and is
never rounded to bf16; the NVFP4 activation tensor scale is taken over the
whole x [T, H] and over the whole h [T*k, I]; y is float32-comparable float64.
"""
from __future__ import annotations

import math

import numpy as np

from . import quant
from .formats import bf16_to_f64, unpack_nibbles


def permute(topk_ids, num_experts: int):
    """Stable sort of the T*k (token, slot) pairs by expert.

    Pair p = t*k + j.  Returns (offsets [E+1], pair_of_row [T*k],
    row_of_pair [T*k]): rows offsets[e]..offsets[e+1]-1 belong to expert e and
    hold that expert's pairs in increasing pair order."""
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= num_experts):
        raise ValueError("expert id out of range")
    pair_of_row = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row_of_pair = np.empty_like(pair_of_row)
    row_of_pair[pair_of_row] = np.arange(flat.size)
    return offsets, pair_of_row, row_of_pair


def route(logits, bias, k: int):
    """Top-k routing of T tokens over E experts (the caller's step in front of
    the layer; routing width k a runtime value, FP4-Local-AZ card, "What is
    different from NVIDIA's checkpoint").

    Reading: l'_e = fp32(logit_e + bias_e); the experts in order of
    decreasing l', equal values by increasing id; the first k; weights the
    softmax over those k l' (the renormalized top-k softmax) in float64 with
    an exactly rounded sum, rounded to float32.  Returns (ids int32 [T, k],
    weights float32 [T, k])."""
    lp = np.asarray(logits, dtype=np.float32)
    T, E = lp.shape
    if not 1 <= k <= E:
        raise ValueError("k outside [1, E]")
    if bias is not None:
        lp = (lp + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    eid = np.broadcast_to(np.arange(E), lp.shape)
    order = np.lexsort((eid, -lp), axis=-1)[:, :k]  # primary key -l', then the id
    ids = order.astype(np.int32)
    w = np.empty((T, k), np.float32)
    for t in range(T):
        sel = [float(lp[t, e]) for e in order[t]]
        z = [math.exp(v - sel[0]) for v in sel]
        tot = math.fsum(z)
        w[t] = [np.float32(v / tot) for v in z]
    return ids, w


def silu(v):
    """SiLU(v) = v * sigmoid(v), the gate activation of the SwiGLU experts
    (FP4-Local AZ card, "The shared expert": silu(0) * 0 = 0)."""
    return v / (1.0 + np.exp(-v))


def sigmoid(v):
    """Logistic sigmoid 1 / (1 + e^-v): the shared expert's per-token gate
    (FP4-Local AZ card, "The shared expert")."""
    return 1.0 / (1.0 + np.exp(-v))


# ---------------------------------------------------------------- weights

def quantize_expert_weight(w_bits, w_fmt: str, rule: str = "4over6"):
    """Quantize one expert matrix given as bf16 bits [out, in]."""
    w = bf16_to_f64(w_bits)
    if w_fmt == "nvfp4":
        return quant.quantize_nvfp4(w, rule)
    if w_fmt == "mxfp4":
        return quant.quantize_mxfp4(w, rule)
    if w_fmt == "fp8_block":
        return quant.quantize_fp8_block_weight(w)
    if w_fmt == "mxfp8":
        return quant.quantize_mxfp8(w)
    raise ValueError(w_fmt)


def dequantize_weight(q, w_fmt: str) -> np.ndarray:
    """Exact float64 values of a quantized matrix (codes unpacked or packed)."""
    codes = q["codes"]
    if w_fmt == "nvfp4":
        return quant.dequantize_nvfp4(codes, q["scales"], q["tensor_scale"])
    if w_fmt == "mxfp4":
        return quant.dequantize_mxfp4(codes, q["scales"])
    if w_fmt == "fp8_block":
        return quant.dequantize_fp8_block_weight(codes, q["scales"])
    if w_fmt == "mxfp8":
        return quant.dequantize_mxfp8(codes, q["scales"])
    raise ValueError(w_fmt)


def unpacked(q):
    """Copy of a quantized record with 4-bit codes unpacked (if they are packed)."""
    return dict(q, codes=unpack_nibbles(q["codes"]))


# ------------------------------------------------------------ activations

def quantize_activation(v, a_fmt: str):
    """Dynamic activation quantization; returns (exact dequantized values, record)."""
    v = np.asarray(v, dtype=np.float64)
    if a_fmt == "none":
        return v, None
    if a_fmt == "nvfp4":
        q = quant.quantize_nvfp4(v, "rtn")
        return quant.dequantize_nvfp4(q["codes"], q["scales"], q["tensor_scale"]), q
    if a_fmt == "mxfp8":
        q = quant.quantize_mxfp8(v)
        return quant.dequantize_mxfp8(q["codes"], q["scales"]), q
    if a_fmt in ("fp8_row", "fp8_block"):
        q = quant.quantize_fp8_rows(v)
        return quant.dequantize_fp8_rows(q["codes"], q["scales"]), q
    raise ValueError(a_fmt)


# ------------------------------------------------------------------ layer

def moe_forward(layer, x_bits, topk_ids, topk_weights, sample_tokens=None,
                return_stages: bool = False):
    """Routed-expert FFN in float64.

    layer: dict with
      w_fmt, a_fmt, num_experts, hidden, inter,
      w13(e) -> quantized record of expert e's fused gate_up [2I, H] (codes unpacked),
      w2(e)  -> quantized record of expert e's down [H, I],
      optional shared: dict(w13=record [2S, H] MXFP8, w2=record [H, S] MXFP8,
                            gate_bits=bf16 bits [H]).
    x_bits: bf16 bits [T, H]; topk_ids int [T, k]; topk_weights float [T, k].
    sample_tokens: optional token indices; y is returned for those rows only.
      With NVFP4 activations the tensor scale of h needs every pair's h, so
      all pairs' gate_up outputs are still computed.
    """
    w_fmt, a_fmt = layer["w_fmt"], layer["a_fmt"]
    E, I = layer["num_experts"], layer["inter"]
    x = bf16_to_f64(x_bits)
    T, k = np.asarray(topk_ids).shape
    ids = np.asarray(topk_ids, dtype=np.int64)
    wts = np.asarray(topk_weights, dtype=np.float64)
    tokens = np.arange(T) if sample_tokens is None else np.asarray(sample_tokens)

    xq, xrec = quantize_activation(x, a_fmt)
    pairs_needed = np.zeros(T * k, bool)
    if a_fmt == "nvfp4" or sample_tokens is None:
        pairs_needed[:] = True
    else:
        for t in tokens:
            pairs_needed[t * k:(t + 1) * k] = True

    offsets, pair_of_row, _ = permute(ids, E)
    h = np.zeros((T * k, I))
    for e in range(E):
        rows = pair_of_row[offsets[e]:offsets[e + 1]]
        rows = rows[pairs_needed[rows]]
        if rows.size == 0:
            continue
        w13 = dequantize_weight(layer["w13"](e), w_fmt)
        gu = xq[rows // k] @ w13.T
        h[rows] = silu(gu[:, :I]) * gu[:, I:]

    if a_fmt == "nvfp4":
        hq, hrec = quantize_activation(h, a_fmt)
    else:
        hq = np.zeros_like(h)
        sel = np.nonzero(pairs_needed)[0]
        hq[sel], hrec = quantize_activation(h[sel], a_fmt)

    H = layer["hidden"]
    y = np.zeros((len(tokens), H))
    tok_pos = {int(t): i for i, t in enumerate(tokens)}
    for e in range(E):
        rows = pair_of_row[offsets[e]:offsets[e + 1]]
        rows = np.array([p for p in rows if int(p // k) in tok_pos], dtype=np.int64)
        if rows.size == 0:
            continue
        w2 = dequantize_weight(layer["w2"](e), w_fmt)
        o = hq[rows] @ w2.T
        for r, p in enumerate(rows):
            t, j = divmod(int(p), k)
            y[tok_pos[t]] += wts[t, j] * o[r]

    shared = layer.get("shared")
    if shared is not None:
        y += shared_forward(shared, x[tokens])

    if return_stages:
        return y, {"h": h, "hq": hq, "xq": xq, "xrec": xrec, "hrec": hrec,
                   "offsets": offsets, "pair_of_row": pair_of_row}
    return y


def shared_forward(shared, x) -> np.ndarray:
    """sigmoid(x . w_g) * Down_s(SiLU(G_s x~) * U_s x~), x~ and h dynamic MXFP8."""
    S = shared["w13"]["codes"].shape[0] // 2
    xq, _ = quantize_activation(x, "mxfp8")
    w13 = dequantize_weight(shared["w13"], "mxfp8")
    gu = xq @ w13.T
    h = silu(gu[:, :S]) * gu[:, S:]
    hq, _ = quantize_activation(h, "mxfp8")
    o = hq @ dequantize_weight(shared["w2"], "mxfp8").T
    gate = sigmoid(x @ bf16_to_f64(shared["gate_bits"]))
    return gate[:, None] * o


def dense_swiglu(x, w13, w2):
    """Plain SwiGLU y = W2 (SiLU(Wg x) * Wu x) on float64 matrices (for pins)."""
    I = w13.shape[0] // 2
    gu = x @ w13.T
    return (silu(gu[:, :I]) * gu[:, I:]) @ w2.T
