"""The synthetic workloads of the ternary linear layer (shapes, formats, scales).

Shapes follow a LLaMA-style block at hidden size 4096 and MLP size 11008 for
decode, and an 8192 / 28672 projection pair for prefill.  Weights are stored
out x in (N x K); activations are M x K fp16.
"""
FMT_2BIT = 0
FMT_1P6BIT = 1
FMT_NAMES = {FMT_2BIT: "2bit", FMT_1P6BIT: "1.6bit"}

# workload 1: one small layer, both formats, fixed scale 0.02
SMALL = dict(workload_id=1, M=1, K=512, N=256, scale=0.02, fmts=(FMT_2BIT, FMT_1P6BIT))

# workload 2: decode GEMV at M=1, 2-bit, scale ~ U(0.01, 0.05); the three shapes of a block
DECODE_SHAPES = [  # (name, K, N)
    ("attn_proj_4096x4096", 4096, 4096),
    ("gate_up_4096to11008", 4096, 11008),
    ("down_11008to4096", 11008, 4096),
]
DECODE = dict(workload_id=2, M=1, shapes=DECODE_SHAPES, fmt=FMT_2BIT)

# workload 3: batched decode, M in {4, 8, 16}, both formats
BATCHED = dict(workload_id=3, Ms=(4, 8, 16),
               shapes=[("gate_up_4096to11008", 4096, 11008), ("down_11008to4096", 11008, 4096)],
               fmts=(FMT_2BIT, FMT_1P6BIT))

# workload 6: a middling number of rows (large-batch decode, short prefill chunks), 2-bit, on the
# kernel family tri_linear picks (the small-M kernels over 16-row slices, or the GEMM)
MID_M = dict(workload_id=6, Ms=(32, 64, 128, 256),
             shapes=[("gate_up_4096to11008", 4096, 11008), ("down_11008to4096", 11008, 4096)], fmt=FMT_2BIT)

# workload 7: decode on the prefill matrices (a 70B-class MLP, 58.7 MB packed 2-bit per
# matrix), M in {1, 2}, both formats: launches long enough for the streaming rate to dominate
DECODE_LARGE = dict(workload_id=7, Ms=(1, 2),
                    shapes=[("up_8192to28672", 8192, 28672), ("down_28672to8192", 28672, 8192)],
                    fmts=(FMT_2BIT, FMT_1P6BIT))

# workload 4: one LLaMA-style block decode step (seven ternary linears), M in {1, 8}
BLOCK_LAYERS = [  # (name, K, N)
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 4096, 11008), ("up", 4096, 11008), ("down", 11008, 4096),
]
BLOCK = dict(workload_id=4, Ms=(1, 8), layers=BLOCK_LAYERS, fmt=FMT_2BIT, hidden=4096, mlp=11008,
             rms_eps=1e-5)

# workload 5: prefill GEMM, M = 2048, scale 0.015, 2-bit then 1.6-bit
PREFILL = dict(workload_id=5, M=2048, shapes=[("up_8192to28672", 8192, 28672), ("down_28672to8192", 28672, 8192)],
               scale=0.015, fmts=(FMT_2BIT, FMT_1P6BIT))
