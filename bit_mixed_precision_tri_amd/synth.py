"""Seeded synthetic inputs for the ternary linear layer.

This module only draws random numbers: it holds none of the layer's arithmetic,
so both the HIP path and the CPU oracle may use it.  Every draw comes from
numpy's PCG64 generator seeded with ``[workload_id, layer_id, stream_id]``
(stream 0 = weights, 1 = activations, 2 = scale, 3 = latent weights).

Distributions (the ternary linear layer of a TriLM, weights in {-1, 0, +1}
times one shared fp32 scale, fp16 activations):
  * trits: P(-1) = P(+1) = 0.3, P(0) = 0.4, int8, one (N, K) matrix per layer;
  * activations: N(0, 1) drawn in float32 and rounded to fp16 (round to nearest even);
  * scale: a fixed value, or U(0.01, 0.05) rounded to fp32;
  * latent (full-precision) weights for the quantiser: N(0, std^2) in float32, std 0.02 by
    default (a common initialisation scale of transformer linear layers).
"""
import numpy as np

STREAM_W, STREAM_X, STREAM_SCALE, STREAM_LATENT = 0, 1, 2, 3


def rng_for(workload_id, layer_id, stream_id):
    return np.random.default_rng([int(workload_id), int(layer_id), int(stream_id)])


def trits(rng, N, K, p_neg=0.3, p_zero=0.4, chunk_rows=1024):
    """(N, K) int8 with P(-1)=p_neg, P(0)=p_zero, P(+1)=1-p_neg-p_zero (drawn row-chunk by row-chunk)."""
    out = np.empty((N, K), dtype=np.int8)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        u = rng.random((r1 - r0, K), dtype=np.float32)
        blk = np.ones((r1 - r0, K), dtype=np.int8)
        blk[u < p_neg + p_zero] = 0
        blk[u < p_neg] = -1
        out[r0:r1] = blk
    return out


def activations(rng, M, K):
    """(M, K) float16 ~ N(0, 1), drawn in float32 then rounded to fp16."""
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def uniform_scale(rng, lo=0.01, hi=0.05):
    return float(np.float32(rng.uniform(lo, hi)))


def layer_inputs(workload_id, layer_id, M, N, K, scale=None):
    """Trits W (N, K), activations X (M, K) and the fp32 scale for one layer."""
    W = trits(rng_for(workload_id, layer_id, STREAM_W), N, K)
    X = activations(rng_for(workload_id, layer_id, STREAM_X), M, K)
    s = float(np.float32(scale)) if scale is not None else uniform_scale(rng_for(workload_id, layer_id, STREAM_SCALE))
    return W, X, s


def latent_weights(rng, N, K, std=0.02, chunk_rows=1024):
    """(N, K) float32 ~ N(0, std^2), drawn in float32 row-chunk by row-chunk."""
    out = np.empty((N, K), dtype=np.float32)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        out[r0:r1] = rng.standard_normal((r1 - r0, K), dtype=np.float32)
    out *= np.float32(std)
    return out
