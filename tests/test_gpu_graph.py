"""HIP graph capture of the library's launches (how bench.py times a decode step): a graph holding
every kernel family is replayed several times, with new inputs written by ordinary eager work
between the replays, and every replay's outputs must equal those of the same calls made eagerly,
bit for bit (the kernels are deterministic and read their inputs through fixed pointers)."""
import numpy as np
import pytest

import bit_mixed_precision_tri_amd as tri
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu
F2, F16 = tri.TRI_FMT_2BIT, tri.TRI_FMT_1P6BIT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tri.lib()
    yield
    torch.cuda.synchronize()


def test_graph_replays_equal_eager_calls():
    import torch
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(77)

    def trits(n, k):
        return torch.randint(-1, 2, (n, k), dtype=torch.int8, device=dev, generator=g)

    # (M, N, K, fmt): M = 1 decode, batched, sliced middling M, the GEMM (full and quarter tiles)
    layers = [(1, 4096, 4096, F2), (1, 2000, 3000, F16), (8, 3000, 4096, F2), (40, 1000, 1000, F16),
              (300, 1100, 512, F2), (2048, 600, 256, F16)]
    Ws = [tri.pack(trits(n, k), f) for (_, n, k, f) in layers]
    Xs = [torch.empty((m, k), dtype=torch.float16, device=dev) for (m, _, k, _) in layers]
    Ys = [torch.empty((m, n), dtype=torch.float16, device=dev) for (m, n, _, _) in layers]
    # a grouped launch and a fused one (norm with gain, residual; the gate/up pair)
    Kg = 1024
    Wg = [tri.pack(trits(n, Kg), F2) for n in (512, 512, 256)]
    Xg = torch.empty((4, Kg), dtype=torch.float16, device=dev)
    Yg = [torch.empty((4, n), dtype=torch.float16, device=dev) for n in (512, 512, 256)]
    gain = torch.empty(Kg, dtype=torch.float16, device=dev)
    Rf = torch.empty((4, 512), dtype=torch.float16, device=dev)
    Yf = [torch.empty((4, 512), dtype=torch.float16, device=dev) for _ in range(2)]
    Yp = torch.empty((4, 512), dtype=torch.float16, device=dev)
    # the quantiser
    Wl = torch.empty((700, 900), dtype=torch.float32, device=dev)
    Wq = torch.empty((700, tri.tri_row_bytes(900, F16)), dtype=torch.uint8, device=dev)
    sq = torch.empty(1, dtype=torch.float32, device=dev)
    nws = tri.tri_quantize_workspace_bytes(700, 900)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def step():
        for (m, n, k, f), X, Wp, Y in zip(layers, Xs, Ws, Ys):
            tri.tri_linear(X, Wp, 0.02, m, n, k, f, Y)
        tri.tri_linear_grouped(Xg, Wg, [0.02, -0.03, 0.04], 4, [512, 512, 256], Kg, F2, Yg)
        tri.tri_linear_fused(Xg, Wg[:2], [0.02, -0.03], 4, [512, 512], Kg, F2, Yf, norm=True, gain=gain,
                             residuals=[Rf, None])
        tri.tri_linear_fused(Xg, Wg[:2], [0.02, -0.03], 4, [512, 512], Kg, F2, [Yp, None], norm=True, pair=True)
        tri.tri_quantize(Wl, 700, 900, F16, Wq, sq, ws, nws)

    outs = lambda: [t.clone() for t in Ys + Yg + Yf + [Yp, Wq, sq]]

    def new_inputs():
        for X in Xs + [Xg, Rf]:
            X.copy_((torch.randn(X.shape, device=dev, generator=g) * 0.5).half())
        gain.copy_((1 + 0.1 * torch.randn(Kg, device=dev, generator=g)).half())
        Wl.copy_(0.02 * torch.randn(Wl.shape, device=dev, generator=g))

    new_inputs()
    step()                                       # (first calls outside capture)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.synchronize()
    for r in range(3):
        new_inputs()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outs()
        step()                                   # the same calls, eagerly, on the same inputs
        torch.cuda.synchronize()
        want = outs()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), "replay %d, output %d differs from the eager call" % (r, i)
        say("graph replay %d: %d outputs equal the eager calls" % (r, len(got)))
    del graph
