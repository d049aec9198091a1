"""w4a8_gemm_fused_act_noalloc (the entry point on the library's static
per-GPU scratch) against w4a8_gemm_fused_act with a workspace, through the C
ABI: same outputs bit for bit, and the INT32 sums equal to the oracle's, on
several calls in a row that reuse the one scratch array with ever smaller
inputs."""
import numpy as np
import pytest

import oracle as O
from gemv_nibble_unpack_amd import workloads as WL
from tests._helpers import say

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_nibble_unpack_amd as G
    G.load()
    return G


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# in call order: the prefill configuration (two launches; the int8 rows take
# 8 MiB of the scratch), a smaller two-launch shape, a decode shape split over
# K (arrival counters and partial sums in the scratch), and a decode shape
# that quantizes in the kernel's prologue (no scratch)
CALLS = [(2048, 11008, 4096, np.float16), (40, 300, 512, np.float32),
         (1, 256, 4096, np.float16), (1, 4096, 4096, np.float16)]


def test_noalloc_matches_the_workspace_entry_point(g):
    for i, (M, N, K, dt) in enumerate(CALLS):
        say(f"case noalloc call {i}: M={M} N={N} K={K} {dt.__name__}")
        need = g.w4_fused_act_workspace_bytes(g.W4_LAYOUT_W4A8, M, N, K)
        assert need <= g.W4_NOALLOC_SCRATCH_BYTES
        W = WL.weights_f32(N, K, seed=19000 + i)
        A = WL.activations(M, K, seed=19100 + i, dtype=dt)
        bias = dev(WL.bias_f16(N, seed=19200 + i))
        Wq, ws, _ = g.quantize_pack_w4(dev(W), g.W4_SYM_PER_CHANNEL)
        Wp = g.prepack_w(g.W4_LAYOUT_W4A8, Wq, N, K)
        Ad = dev(A)
        for out, b in ((g.W4_OUT_I32, None), (g.W4_OUT_F16, bias)):
            ref = host(g.w4a8_gemm_fused_act(Ad, Wp, ws, N, bias=b, out_dtype=out))
            got = host(g.w4a8_gemm_fused_act_noalloc(Ad, Wp, ws, N, bias=b, out_dtype=out))
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), (i, out)
            if out == g.W4_OUT_I32:
                qa, _, _ = O.quantize_a8(A)
                qw, _ = O.quantize_w4_sym(W)
                assert np.array_equal(got, O.int_accumulate_f64(qa, qw).astype(np.int32)), i


def test_noalloc_refuses_a_shape_beyond_the_scratch(g):
    M, N, K = 4096, 256, 16384
    assert g.w4_fused_act_workspace_bytes(g.W4_LAYOUT_W4A8, M, N, K) > g.W4_NOALLOC_SCRATCH_BYTES
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    Wp = torch.zeros(g.prepack_bytes(g.W4_LAYOUT_W4A8, N, K), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(N, dtype=torch.float32, device="cuda")
    with pytest.raises(g.W4Error) as e:
        g.w4a8_gemm_fused_act_noalloc(A, Wp, ws, N)
    assert e.value.status == g.W4_ERR_SCRATCH
