"""Process-pool task for the GPU tests' oracle side: the oracle's
quantization of one expert (kept free of torch, so spawned workers import
only numpy and the oracle)."""


def quantize_expert_pair(task):
    """Oracle quantization of one expert's W13 and W2."""
    from oracle import moe
    w13_bits, w2_bits, w_fmt, rule = task
    return moe.quantize_expert_weight(w13_bits, w_fmt, rule), moe.quantize_expert_weight(w2_bits, w_fmt, rule)
