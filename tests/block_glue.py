"""CPU glue of one LLaMA-style decode block around its seven ternary linears
(test infrastructure: the same fp32 code runs between GPU linears and between
oracle linears).

Each of the M activation rows is an independent sequence at its first decode
position, so attention over the single key has softmax weight 1 and returns V;
Q and K are still computed (and checked) but do not change the output:
  h   = x + O(V(rmsnorm(x)))
  out = h + down(silu(gate(rmsnorm(h))) * up(rmsnorm(h)))
RMSNorm has unit gain and eps = 1e-5.  Glue runs in fp32; every linear input is
rounded to fp16 (round to nearest even) first.
"""
import numpy as np


def rmsnorm(x, eps=1e-5):
    x = x.astype(np.float32)
    return (x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + np.float32(eps))).astype(np.float32)


def silu(x):
    x = x.astype(np.float32)
    return (x / (np.float32(1) + np.exp(-x))).astype(np.float32)


def fp16(x):
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def block_step(x, linear):
    """Run the block; `linear(name, X_fp16) -> Y (fp16)`.  Returns (out fp32, {name: input fp16})."""
    inputs = {}

    def lin(name, a):
        inputs[name] = a
        return linear(name, a).astype(np.float32)

    x = x.astype(np.float32)
    a = fp16(rmsnorm(x))
    lin("q", a)
    lin("k", a)
    v = lin("v", a)
    h = x + lin("o", fp16(v))
    b = fp16(rmsnorm(h))
    gate = lin("gate", b)
    up = lin("up", b)
    out = h + lin("down", fp16(silu(gate) * up))
    return out, inputs
