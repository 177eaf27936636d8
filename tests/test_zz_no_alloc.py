"""tri_quantize_noalloc (the quantiser with its partial sums in the library's static device
scratch) against tri_quantize with a caller-owned workspace, through the C ABI: the same packed
bytes and the same scale, bit for bit, on two calls in a row (the second on a smaller matrix,
after the first has filled most of the scratch), both also checked against the oracle."""
import numpy as np
import pytest

import oracle
import bit_mixed_precision_tri_amd as tri
from bit_mixed_precision_tri_amd import synth
from tests.gpu_helpers import say, cuda, host

pytestmark = pytest.mark.gpu
FMTS = (tri.TRI_FMT_2BIT, tri.TRI_FMT_1P6BIT)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tri.lib()
    yield
    torch.cuda.synchronize()


def with_workspace(Wd, N, K, fmt):
    import torch
    Wp = torch.empty((N, tri.tri_row_bytes(K, fmt)), dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    nb = tri.tri_quantize_workspace_bytes(N, K)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    tri.tri_quantize(Wd, N, K, fmt, Wp, s, ws, nb)
    return host(Wp), host(s)


def without_workspace(Wd, N, K, fmt):
    import torch
    Wp = torch.full((N, tri.tri_row_bytes(K, fmt)), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    tri.tri_quantize_noalloc(Wd, N, K, fmt, Wp, s)
    return host(Wp), host(s)


@pytest.mark.parametrize("fmt", FMTS)
def test_noalloc_equals_workspace_variant(fmt):
    assert tri.tri_quantize_workspace_bytes(2000, 4096) <= tri.TRI_QUANTIZE_SCRATCH_BYTES
    rng = synth.rng_for(990, fmt, synth.STREAM_LATENT)
    # 2000 x 4096 fills 2000 of the 2048 partial sums; 37 x 301 then needs 11 (stale sums beyond)
    for (N, K) in [(2000, 4096), (37, 301)]:
        W = synth.latent_weights(rng, N, K)
        Wd = cuda(W)
        say("noalloc quantize N=%d K=%d fmt=%d" % (N, K, fmt))
        Wp0, s0 = without_workspace(Wd, N, K, fmt)
        Wp1, s1 = with_workspace(Wd, N, K, fmt)
        np.testing.assert_array_equal(Wp0, Wp1, err_msg="bytes N=%d K=%d" % (N, K))
        assert s0.view(np.uint32)[0] == s1.view(np.uint32)[0], (s0, s1)
        T_ref, s_ref = oracle.quantize(W)
        assert abs(float(s0[0]) - float(s_ref)) <= float(np.spacing(s_ref)), (s0, s_ref)
        if np.float32(s0[0]) == np.float32(s_ref):
            np.testing.assert_array_equal(Wp0, oracle.pack(T_ref, fmt))
